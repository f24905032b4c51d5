// k_sample.hip -- rejection-sampling acceptance of a point-mass draft chain,
// for gfx950.
//
// Rule (colibri "MTP speculative decoding and prefetch" s5): with
// p_j = softmax(logits[j] / temperature), draft token d_j is kept while
// u_j < p_j(d_j); at the first rejection n the output token is drawn from
// p_n with d_n removed and the rest renormalised, or from p_T when every
// draft is kept.  The draw is the smallest index i whose cumulative mass, in
// index order with the removed token counting zero, exceeds u_T times the
// remaining total mass.  Uniforms are inputs.
//
// Two launches.  (1) k_softmax_part: every logits row is cut into chunks of
// kSampleChunk elements; a wave streams one chunk in 16-byte loads and keeps
// an online (max, sum of exp(z - max)) per lane, z = logit / temperature,
// then reduces them.  (2) k_sample_walk: one workgroup per
// sequence merges each row's partials into (m, Z), takes the acceptance
// decisions, scans the chunk masses of the output row (the removed token
// subtracted) to find the chunk where the cumulative mass crosses the
// threshold, and rescans that chunk only: each thread sums 16 consecutive
// elements in order, a block scan finds the thread whose range holds the
// crossing, and that thread walks its 16 elements in the same order, so the
// two levels agree on every partial sum.  Logits must be finite.

#include <algorithm>

#include "gdn_common.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

constexpr int kNT = 256;

// Merge (m2, s2) into (m, s): both are (max, sum of exp(z - max)) pairs.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -__builtin_inff()) return;  // both empty
  s = s * __expf(m - M) + s2 * __expf(m2 - M);
  m = M;
}

__device__ __forceinline__ void wave_lse(float& m, float& s) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave);
    const float s2 = __shfl_xor(s, off, kWave);
    lse_merge(m, s, m2, s2);
  }
}

template <int ESZ>
__device__ __forceinline__ float logit(const SampleArgs& p, size_t row, int i) {
  return ESZ == 2 ? ld_in(static_cast<const uint16_t*>(p.logits) + row * p.V, i)
                  : ld_in(static_cast<const float*>(p.logits) + row * p.V, i);
}

// One wave per chunk: lane l takes 16-byte vectors l, l + 64, ... of its
// chunk (all loads in flight at once), then the wave reduces.  Waves stride
// over the (row, chunk) pairs of the whole batch, so the grid stays a few
// thousand workgroups however many chunks there are.
template <int ESZ>
__global__ __launch_bounds__(kNT) void k_softmax_part(SampleArgs p) {
  constexpr int EPV = 16 / ESZ;                           // elements per 16-byte vector
  constexpr int VPL = kSampleChunk / EPV / kWave;         // vectors per lane per chunk
  constexpr int NWV = kNT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const float it = p.inv_tau;
  const float c = it * 1.44269504088896341f;  // exp(z - m) = exp2(x c - mx c), z = x / tau
  const size_t V = p.V;
  const long long total = static_cast<long long>(p.B) * (p.T + 1) * p.split;
  const bool vec = ((V * ESZ) % 16) == 0;
  for (long long q = static_cast<long long>(blockIdx.x) * NWV + wave; q < total;
       q += static_cast<long long>(gridDim.x) * NWV) {
    const size_t row = q / p.split;
    const int part = static_cast<int>(q % p.split);
    const int beg = part * kSampleChunk;
    const int end = min(beg + kSampleChunk, p.V);
    float m = -__builtin_inff(), s = 0.f;
    if (vec) {
      // chunk starts are multiples of 8 elements, so vectors stay aligned;
      // the running max mx is kept in logit units
      const uint4* vp = reinterpret_cast<const uint4*>(static_cast<const char*>(p.logits) + row * V * ESZ);
      const int vbeg = beg / EPV, vend = end / EPV;
      uint4 w[VPL];
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        const int v = vbeg + lane + k * kWave;
        w[k] = vp[v < vend ? v : vbeg];
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        if (vbeg + lane + k * kWave >= vend) continue;
        const uint32_t ws[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
        float x[EPV];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          if (ESZ == 2) {
            x[2 * h] = __uint_as_float(ws[h] << 16);
            x[2 * h + 1] = __uint_as_float(ws[h] & 0xffff0000u);
          } else {
            x[h] = __uint_as_float(ws[h]);
          }
        }
        float vm = x[0];
#pragma unroll
        for (int e = 1; e < EPV; ++e) vm = fmaxf(vm, x[e]);
        if (vm > mx) {
          s *= __builtin_amdgcn_exp2f((mx - vm) * c);
          mx = vm;
        }
        const float nmc = -mx * c;
#pragma unroll
        for (int e = 0; e < EPV; ++e) s += __builtin_amdgcn_exp2f(fmaf(x[e], c, nmc));
      }
      m = mx * it;  // back to z units (-inf stays -inf)
      for (int i = vend * EPV + lane; i < end; i += kWave) lse_merge(m, s, logit<ESZ>(p, row, i) * it, 1.f);
    } else {
      for (int i = beg + lane; i < end; i += kWave) lse_merge(m, s, logit<ESZ>(p, row, i) * it, 1.f);
    }
    wave_lse(m, s);
    if (lane == 0) {
      p.part_m[q] = m;
      p.part_s[q] = s;
    }
  }
}

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ float wave_scan(float v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float y = __shfl_up(v, off, kWave);
    if (lane >= off) v += y;
  }
  return v;
}

template <int ESZ>
__global__ __launch_bounds__(kNT) void k_sample_walk(SampleArgs p) {
  constexpr int NWV = kNT / kWave;
  __shared__ float s_rm[65], s_rz[65];  // per row: max and total of exp(z - max)
  __shared__ float s_wf[NWV];
  __shared__ int s_wi[NWV];
  __shared__ int s_chunk;
  __shared__ float s_rem;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int bb = blockIdx.x;
  const int T = p.T, V = p.V, split = p.split;
  const int rows = T + 1;
  const float it = p.inv_tau;
  const size_t row0 = static_cast<size_t>(bb) * rows;

  // (1) each row's (m, Z) from its chunk partials
  for (int r = wave; r < rows; r += NWV) {
    float m = -__builtin_inff(), s = 0.f;
    for (int c = lane; c < split; c += kWave)
      lse_merge(m, s, p.part_m[(row0 + r) * split + c], p.part_s[(row0 + r) * split + c]);
    wave_lse(m, s);
    if (lane == 0) {
      s_rm[r] = m;
      s_rz[r] = s;
    }
  }
  __syncthreads();

  // (2) acceptance: n = first j with u_j >= p_j(d_j)
  const int* draft = p.draft + static_cast<size_t>(bb) * T;
  const float* u = p.uniforms + static_cast<size_t>(bb) * rows;
  int first = T, bad = 0;
  for (int j = tid; j < T; j += kNT) {
    const int d = draft[j];
    bool keep = false;
    if (d >= 0 && d < V) {
      const float pd = __expf(logit<ESZ>(p, row0 + j, d) * it - s_rm[j]) / s_rz[j];
      keep = u[j] < pd;
    } else {
      bad = 1;
    }
    if (!keep) first = min(first, j);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    first = min(first, __shfl_xor(first, off, kWave));
    bad |= __shfl_xor(bad, off, kWave);
  }
  if (lane == 0) s_wi[wave] = first;
  if (bad && lane == 0 && p.dev_err) atomicOr(p.dev_err, GDN_DEV_ERR_TOKEN);
  __syncthreads();
  int n = s_wi[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) n = min(n, s_wi[w]);

  // (3) output row n: mass left after removing the rejected token
  const size_t orow = row0 + n;
  const int dn = n < T ? draft[n] : -1;
  const int ban = (dn >= 0 && dn < V) ? dn : -1;
  const float m = s_rm[n];
  const float eb = ban >= 0 ? __expf(logit<ESZ>(p, orow, ban) * it - m) : 0.f;
  const float target = u[T] * fmaxf(s_rz[n] - eb, 0.f);
  // chunk where the cumulative mass first exceeds the target (wave 0, in order)
  if (wave == 0) {
    float run = 0.f;
    int chosen = -1, last_pos = 0;
    float before_last = 0.f;
    for (int c0 = 0; c0 < split && chosen < 0; c0 += kWave) {
      const int c = c0 + lane;
      float w = 0.f;
      if (c < split) {
        w = p.part_s[orow * split + c] * __expf(p.part_m[orow * split + c] - m);
        if (ban >= c * kSampleChunk && ban < (c + 1) * kSampleChunk) w = fmaxf(w - eb, 0.f);
      }
      const float incl = wave_scan(w, lane);
      const unsigned long long hit = __ballot(c < split && run + incl > target);
      const unsigned long long pos = __ballot(c < split && w > 0.f);
      if (hit) {
        const int lf = __builtin_ctzll(hit);
        chosen = c0 + lf;
        run += __shfl(incl - w, lf, kWave);
      } else {
        if (pos) {
          const int ll = 63 - __builtin_clzll(pos);
          last_pos = c0 + ll;
          before_last = run + __shfl(incl - w, ll, kWave);
        }
        run += __shfl(incl, kWave - 1, kWave);
      }
    }
    if (chosen < 0) {  // rounding left the target above the total: last chunk with mass
      chosen = last_pos;
      run = before_last;
    }
    if (lane == 0) {
      s_chunk = chosen;
      s_rem = target - run;
    }
  }
  __syncthreads();

  // (4) rescan the chosen chunk: 16 consecutive elements per thread
  const int beg = s_chunk * kSampleChunk + 16 * tid;
  const float rem = s_rem;
  float ev[16];
  float sum = 0.f;
  int lastp = -1;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int i = beg + e;
    float x = 0.f;
    if (i < V && i < (s_chunk + 1) * kSampleChunk && i != ban) x = __expf(logit<ESZ>(p, orow, i) * it - m);
    ev[e] = x;
    sum += x;
    if (x > 0.f) lastp = i;
  }
  // exclusive block scan of the thread sums
  const float incl = wave_scan(sum, lane);
  if (lane == kWave - 1) s_wf[wave] = incl;
  __syncthreads();
  float excl = incl - sum;
  for (int w = 0; w < wave; ++w) excl += s_wf[w];
  int pick = -1;
  if (excl <= rem && excl + sum > rem) {
    float run = excl;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      run += ev[e];
      if (pick < 0 && run > rem) pick = beg + e;
    }
  }
  // at most one thread holds the crossing; otherwise the last index with mass
  int key = pick >= 0 ? (1 << 30) + pick : lastp;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) key = max(key, __shfl_xor(key, off, kWave));
  __syncthreads();
  if (lane == 0) s_wi[wave] = key;
  __syncthreads();
  if (tid == 0) {
    int k = s_wi[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) k = max(k, s_wi[w]);
    const int tok = k >= (1 << 30) ? k - (1 << 30) : (k >= 0 ? k : (ban >= 0 ? ban : 0));
    p.n_keep[bb] = n;
    p.token[bb] = tok;
  }
  int* path = p.path + static_cast<size_t>(bb) * T;
  for (int j = tid; j < T; j += kNT) path[j] = j < n ? j : -1;
}

}  // namespace

int sample_split(int V) { return (V + kSampleChunk - 1) / kSampleChunk; }

hipError_t launch_sample(const SampleArgs& a, int dtype, hipStream_t s) {
  const long long chunks = static_cast<long long>(a.B) * (a.T + 1) * a.split;
  if (a.T + 1 > 65) return hipErrorInvalidValue;
  const long long waves = kNT / kWave;
  const long long grid = std::min<long long>((chunks + waves - 1) / waves, 4096);
  if (dtype == 1) {
    hipLaunchKernelGGL(k_softmax_part<2>, dim3(grid), dim3(kNT), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_softmax_part<4>, dim3(grid), dim3(kNT), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == 1)
    hipLaunchKernelGGL(k_sample_walk<2>, dim3(a.B), dim3(kNT), 0, s, a);
  else
    hipLaunchKernelGGL(k_sample_walk<4>, dim3(a.B), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace gdn
