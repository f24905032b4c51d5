// k_accept.hip -- greedy acceptance of a draft chain or draft tree, for gfx950.
//
// Rule (xserv "Phase 25" s2 pseudo-code; colibri "MTP speculative decoding"
// s5): a draft is accepted while it equals the target's argmax at its
// position; the correction (bonus) token is the argmax where the walk stops.
// Trees (tree-aware verify, GDN page s8) walk from the virtual root to the
// lowest-index child whose token equals the current row's argmax.
//
// Two launches.  (1) k_argmax_part: the (T+1) logits rows of every sequence
// are split into `split` chunks so the grid holds enough workgroups to keep
// HBM busy; each workgroup streams its chunk in 16-byte loads and reduces to
// (max value, lowest index).  (2) k_accept_walk: one wave per sequence folds
// the partials into each row's argmax and walks the chain / tree.  Ties at
// every level keep the lowest index, so the result equals a plain sequential
// first-maximum scan.  Infinities compare as values (a row of -inf gives
// index 0); a NaN is never the maximum (it loses every comparison, and the
// "no value yet" seed below loses to any number), so a row with no number
// gives index 0, and a NaN seen in a row sets GDN_DEV_ERR_NAN.  The walk never
// leaves the device.

#include "gdn_common.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

struct Best {
  float v;
  int i;
};

// Seed of every reduction: below or equal to any number, and any number at a
// real index beats it (equal value, lower index); NaN never does.
constexpr int kNoIndex = 0x7fffffff;

// Keep the larger value; on equal values the lower index.
__device__ __forceinline__ Best better(Best a, Best b) {
  return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

__device__ __forceinline__ Best wave_best(Best x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Best o;
    o.v = __shfl_xor(x.v, off, kWave);
    o.i = __shfl_xor(x.i, off, kWave);
    x = better(x, o);
  }
  return x;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int ESZ>
__global__ __launch_bounds__(256) void k_argmax_part(AcceptArgs p) {
  constexpr int NT = 256;
  constexpr int EPV = 16 / ESZ;  // elements per 16-byte vector
  __shared__ Best s_best[NT / kWave];
  __shared__ bool s_nan[NT / kWave];
  const int tid = threadIdx.x;
  const int part = blockIdx.x % p.split;
  const size_t row = blockIdx.x / p.split;
  const size_t V = p.V;
  const int beg = part * p.chunk;
  const int end = min(beg + p.chunk, p.V);
  Best best{-__builtin_inff(), kNoIndex};
  bool nan = false;
  const char* base = static_cast<const char*>(p.logits) + row * V * ESZ;
  if (((V * ESZ) % 16) == 0 && (beg % EPV) == 0) {
    // vector path: 16-byte loads of EPV consecutive elements
    const uint4* vp = reinterpret_cast<const uint4*>(base);
    const int vbeg = beg / EPV;
    const int vend = end / EPV;  // full vectors
    // A thread sees its elements in increasing index order, so an equal
    // value replaces the best only while it is still the seed: the lowest
    // index among equal values is kept.
    auto take = [&](float v, int i) {
      nan |= v != v;
      if (v > best.v || (v == best.v && best.i == kNoIndex)) best = Best{v, i};
    };
    auto scan = [&](const uint4& w, int i0) {
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (ESZ == 2) {
          take(bf16_lo(ws[h]), i0 + 2 * h);
          take(bf16_hi(ws[h]), i0 + 2 * h + 1);
        } else {
          take(__uint_as_float(ws[h]), i0 + h);
        }
      }
    };
    constexpr int U = 8;  // vectors in flight per thread (a whole bf16 chunk in one batch)
    // Every load of a batch is issued before any is scanned; a load past
    // the chunk reads the batch's first vector (a valid address) and is not
    // scanned.
    for (int q = vbeg + tid; q < vend; q += U * NT) {
      uint4 w[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int qj = q + j * NT;
        w[j] = vp[qj < vend ? qj : q];
      }
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (q + j * NT < vend) scan(w[j], (q + j * NT) * EPV);
    }
    for (int i = vend * EPV + tid; i < end; i += NT) {  // ragged tail
      const float v = ESZ == 2 ? ld_in(reinterpret_cast<const uint16_t*>(base), i)
                               : ld_in(reinterpret_cast<const float*>(base), i);
      nan |= v != v;
      best = better(best, Best{v, i});
    }
  } else {
    for (int i = beg + tid; i < end; i += NT) {
      const float v = ESZ == 2 ? ld_in(reinterpret_cast<const uint16_t*>(base), i)
                               : ld_in(reinterpret_cast<const float*>(base), i);
      nan |= v != v;
      best = better(best, Best{v, i});
    }
  }
  best = wave_best(best);
  const bool wave_nan = __any(nan);
  if ((tid & (kWave - 1)) == 0) {
    s_best[tid / kWave] = best;
    s_nan[tid / kWave] = wave_nan;
  }
  __syncthreads();
  if (tid == 0) {
    Best b = s_best[0];
#pragma unroll
    for (int w = 1; w < NT / kWave; ++w) b = better(b, s_best[w]);
    p.part_val[row * p.split + part] = b.v;
    p.part_idx[row * p.split + part] = b.i;
    bool any_nan = false;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) any_nan |= s_nan[w];
    if (any_nan && p.dev_err) atomicOr(p.dev_err, GDN_DEV_ERR_NAN);
  }
}

__global__ __launch_bounds__(64) void k_accept_walk(AcceptArgs p) {
  __shared__ int s_star[65];
  const int lane = threadIdx.x;
  const int bb = blockIdx.x;
  const int T = p.T;
  const int rows = T + 1;
  for (int r = lane; r < rows; r += kWave) {
    const size_t row = static_cast<size_t>(bb) * rows + r;
    Best b{-__builtin_inff(), kNoIndex};
    for (int s = 0; s < p.split; ++s)
      b = better(b, Best{p.part_val[row * p.split + s], p.part_idx[row * p.split + s]});
    s_star[r] = b.i == kNoIndex ? 0 : b.i;  // a row with no number
  }
  __syncthreads();
  const int* draft = p.draft + static_cast<size_t>(bb) * T;
  int* path = p.path + static_cast<size_t>(bb) * T;
  for (int j = lane; j < T; j += kWave) path[j] = -1;
  __syncthreads();
  int n = 0;
  int star = 0;
  if (!p.parent) {
    // longest prefix with draft[j] == argmax(row j)
    int first_bad = T;
    for (int j = lane; j < T; j += kWave)
      if (draft[j] != s_star[j]) first_bad = min(first_bad, j);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) first_bad = min(first_bad, __shfl_xor(first_bad, off, kWave));
    n = first_bad;
    for (int j = lane; j < n; j += kWave) path[j] = j;
    star = s_star[n];
  } else {
    const int* par = p.parent + static_cast<size_t>(bb) * T;
    // validate the parent array (parents precede children)
    int bad = 0;
    for (int v = lane; v < T; v += kWave)
      if (par[v] < -1 || par[v] >= v) bad = 1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) bad |= __shfl_xor(bad, off, kWave);
    if (bad) {
      if (lane == 0) {
        if (p.dev_err) atomicOr(p.dev_err, GDN_DEV_ERR_PARENT);
        p.n_keep[bb] = 0;
        p.bonus[bb] = s_star[0];
      }
      return;
    }
    int cur = -1;
    for (;;) {
      star = s_star[cur + 1];
      // lowest-index child of cur whose token is star
      int cand = T;
      for (int v = lane; v < T; v += kWave)
        if (par[v] == cur && draft[v] == star) cand = min(cand, v);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) cand = min(cand, __shfl_xor(cand, off, kWave));
      if (cand >= T) break;
      if (lane == 0) path[n] = cand;
      ++n;
      cur = cand;
    }
  }
  if (lane == 0) {
    p.n_keep[bb] = n;
    p.bonus[bb] = star;
  }
}

}  // namespace

void accept_split(int B, int T, int V, int* split, int* chunk) {
  const long long rows = static_cast<long long>(B) * (T + 1);
  // At least ~2048 workgroups, and chunks of at most 16384 elements (one
  // batch of eight 16-byte loads per thread for bf16), but of at least 4096;
  // chunk a multiple of 8 so vector loads stay aligned.
  long long sp = (2048 + rows - 1) / rows;
  const long long min_sp = (V + 16383) / 16384;
  if (sp < min_sp) sp = min_sp;
  const long long max_sp = (V + 4095) / 4096;
  if (sp > max_sp) sp = max_sp;
  if (sp < 1) sp = 1;
  long long ch = (V + sp - 1) / sp;
  ch = (ch + 7) / 8 * 8;
  sp = (V + ch - 1) / ch;
  *split = static_cast<int>(sp);
  *chunk = static_cast<int>(ch);
}

hipError_t launch_accept(const AcceptArgs& a, int dtype, hipStream_t s) {
  const long long grid = static_cast<long long>(a.B) * (a.T + 1) * a.split;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (dtype == 1)
    hipLaunchKernelGGL(k_argmax_part<2>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_argmax_part<4>, dim3(grid), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_accept_walk, dim3(a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace gdn
