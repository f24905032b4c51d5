// k_verify_wy.hip -- chunked (WY) verify of a draft chain or draft tree through
// one GDN layer per (layer, sequence, v-head, row block), for gfx950.
//
// The gated delta rule (GDN page s2.1; replay form in s4), per node t with
// parent p (chain: p = t-1; -1 = the committed state S0):
//   S_t = a_t S_p + u_t k_t^T,  u_t = b_t (v_t - a_t S_p k_t),  o_t = S_t q_t.
// Unrolled along each node's ancestor path (products of a along the path):
//   gamma_t = prod of a over t and its ancestors,  Gamma[t,i] = gamma_t/gamma_i
//   u_t + sum_{i in anc(t)} b_t Gamma[t,i] (k_t.k_i) u_i = b_t (v_t - gamma_t S0 k_t)
//   o_t = gamma_t S0 q_t + sum_{i in anc(t) + t} Gamma[t,i] (q_t.k_i) u_i
// so the only products with the state are [K;Q] S0^T -- one dense
// (2T x Dk) x (Dk x Dv) contraction per head, done on fp32 MFMA with S0 read
// once from HBM straight into the B-operand registers.  Everything else is
// O(T * depth * Dv) and runs on the VALU out of LDS.  A tree is the same
// algebra with the ancestor set taken from the parent array (tree-aware
// verify, GDN page s8).  S0 is never written: it stays the pre-verify
// snapshot that rollback replays onto (GDN page s4).
//
// Work decomposition: one 256-thread workgroup per (layer, seq, v-head,
// ROWS-row block of S).  The rows of S are independent recurrences that share
// q, k and the gates, so row blocks need no communication.  Each wave owns
// 16-row column tiles of the MFMA output; lane (c16 = lane%16, kk = lane/16)
// loads S0[row c16][16m + 4kk .. +3] as one float4 per 16-column step m, so a
// wave instruction reads 16 rows x 64 contiguous bytes.

#include "gdn_common.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

constexpr int kMaxK = 8;

template <typename TIn>
__device__ __forceinline__ float conv_at(const VerifyArgs& p, const TIn* x, const TIn* cs,
                                         const int* widx, const float* w, int K, size_t lb,
                                         int ch) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < K) {
      const int idx = widx[j];
      const float xv = idx < 0 ? ld_in(cs, (lb * (K - 1) + (K - 1 + idx)) * p.C + ch)
                               : ld_in(x, (lb * p.T + idx) * p.C + ch);
      acc = fmaf(w[j], xv, acc);
    }
  }
  return p.silu ? acc / (1.f + __expf(-acc)) : acc;
}

template <int DK, int DV, int TMAX, int ROWS, typename TIn>
__global__ __launch_bounds__(256) void k_verify_wy(VerifyArgs p) {
  constexpr int NT = 256;
  constexpr int NWAVE = NT / kWave;
  constexpr int KQ_ROWS = 2 * TMAX;  // k rows [0,TMAX), q rows [TMAX,2TMAX)
  constexpr int KQ_LD = DK + 4;      // +4 floats: conflict-free float4 column reads
  constexpr int WZ_LD = ROWS + 4;
  constexpr int NRB = KQ_ROWS / 16;
  constexpr int NTILE = ROWS / 16;
  constexpr int TPW = (NTILE + NWAVE - 1) / NWAVE;
  constexpr int MSTEPS = DK / 16;
  constexpr int CO_LD = TMAX + 1;
  constexpr int NRBLK = DV / ROWS;
  static_assert(KQ_ROWS % 16 == 0 && ROWS % 16 == 0 && DV % ROWS == 0, "tiling");
  static_assert(KQ_LD >= WZ_LD, "W/Z must fit in the k/q region");

  __shared__ float s_kq[KQ_ROWS * KQ_LD];
  __shared__ float s_A[TMAX * CO_LD];  // b_t Gamma[t,i] k_t.k_i, i proper ancestor of t
  __shared__ float s_O[TMAX * CO_LD];  // Gamma[t,i] q_t.k_i, i ancestor of t or t itself
  __shared__ float s_gam[TMAX], s_ga[TMAX], s_gb[TMAX];
  __shared__ unsigned long long s_anc[TMAX];
  __shared__ int s_par[TMAX];
  __shared__ int s_widx[TMAX * kMaxK];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c16 = lane & 15;
  const int kk = lane >> 4;

  const int G = p.Hv / p.Hk;
  const int n_units = p.L * p.B * p.Hk;
  const UnitSub us = xcd_unit_sub(blockIdx.x, G * NRBLK);
  if (us.unit >= n_units) return;
  const int hk = us.unit % p.Hk;
  const size_t lb = us.unit / p.Hk;  // l * B + b
  const int bb = static_cast<int>(lb % p.B);
  const int l = static_cast<int>(lb / p.B);
  const int g = us.sub / NRBLK;
  const int rblk = us.sub % NRBLK;
  const int hv = hk * G + g;
  const int r0 = rblk * ROWS;
  const int T = p.T;
  const int K = p.K;
  const TIn* x = static_cast<const TIn*>(p.x);
  const TIn* cs = static_cast<const TIn*>(p.conv_state);

  // (1) Issue the state loads first: the long HBM latency overlaps the
  //     conv / norm / Gram prologue below.
  floatx4 sreg[TPW][MSTEPS];
  const float* S_head = p.S + (lb * p.Hv + hv) * static_cast<size_t>(DV * DK);
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int tile = wave + tt * NWAVE;
    if (tile < NTILE) {
      const float* rp = S_head + static_cast<size_t>(r0 + tile * 16 + c16) * DK + 4 * kk;
#pragma unroll
      for (int m = 0; m < MSTEPS; ++m) sreg[tt][m] = *reinterpret_cast<const floatx4*>(rp + 16 * m);
    }
  }

  // (2) Parents (validated), gates, tape g.
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (tid < T) {
    int pv = p.parent ? p.parent[static_cast<size_t>(bb) * T + tid] : tid - 1;
    if (pv < -1 || pv >= tid) {
      s_bad = 1;
      pv = -1;
    }
    s_par[tid] = pv;
    const size_t gi = (lb * T + tid) * p.Hv + hv;
    const TIn* ga = static_cast<const TIn*>(p.a);
    const TIn* gb = static_cast<const TIn*>(p.b);
    const float av = ld_in(ga, gi);
    s_ga[tid] = av;
    s_gb[tid] = ld_in(gb, gi);
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0 && p.dev_err) atomicOr(p.dev_err, GDN_DEV_ERR_PARENT);
    return;
  }
  if (tid < T) {
    if (rblk == 0) p.tg[(lb * T + tid) * p.Hv + hv] = s_ga[tid];
    // conv window of node tid: walk up the ancestors, then old conv rows.
    int cur = tid, old = 0;
    for (int j = K - 1; j >= 0; --j) {
      if (cur >= 0) {
        s_widx[tid * kMaxK + j] = cur;
        cur = s_par[cur];
      } else {
        s_widx[tid * kMaxK + j] = --old;
      }
    }
  }
  if (tid == 0) {
    for (int v = 0; v < T; ++v) {
      const int pv = s_par[v];
      s_anc[v] = pv < 0 ? 0ull : (s_anc[pv] | (1ull << pv));
    }
  }
  __syncthreads();
  if (p.conv_win && l == 0 && hk == 0 && g == 0 && rblk == 0) {
    for (int e = tid; e < T * K; e += NT)
      p.conv_win[static_cast<size_t>(bb) * T * K + e] = s_widx[(e / K) * kMaxK + (e % K)];
  }

  // (3) Conv + SiLU of this k-head's q and k channels for all nodes.
  for (int c = tid; c < 2 * DK; c += NT) {
    const bool isq = c < DK;
    const int cc = isq ? c : c - DK;
    const int ch = isq ? hk * DK + cc : p.Hk * DK + hk * DK + cc;
    const int row0 = isq ? TMAX : 0;
    float w[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      w[j] = j < K ? p.conv_w[(static_cast<size_t>(l) * p.C + ch) * K + j] : 0.f;
    for (int t = 0; t < TMAX; ++t)
      s_kq[(row0 + t) * KQ_LD + cc] = t < T ? conv_at(p, x, cs, s_widx + t * kMaxK, w, K, lb, ch)
                                            : 0.f;
  }
  __syncthreads();

  // (4) L2-normalise the 2T vectors (k rows then q rows), one wave per vector.
  for (int vi = wave; vi < 2 * T; vi += NWAVE) {
    float* r = s_kq + (vi < T ? vi : TMAX + vi - T) * KQ_LD;
    float ss = 0.f;
    for (int e = lane; e < DK; e += kWave) ss = fmaf(r[e], r[e], ss);
    ss = wave_sum(ss);
    const float inv = 1.f / sqrtf(ss + p.eps);
    for (int e = lane; e < DK; e += kWave) r[e] *= inv;
  }
  __syncthreads();

  // Tape k: written once per k-head (by the first v-head's first row block).
  if (g == 0 && rblk == 0) {
    for (int e = tid; e < T * DK; e += NT) {
      const int t = e / DK, c = e % DK;
      p.tk[((lb * T + t) * p.Hk + hk) * DK + c] = s_kq[t * KQ_LD + c];
    }
  }

  // (5) Gram coefficients along each node's ancestor path (one wave per node).
  for (int t = wave; t < T; t += NWAVE) {
    const float* kt = s_kq + t * KQ_LD;
    const float* qt = s_kq + (TMAX + t) * KQ_LD;
    float part = 0.f;
    for (int e = lane; e < DK; e += kWave) part = fmaf(qt[e], kt[e], part);
    const float qk_self = wave_sum(part);
    float gprod = s_ga[t];
    int cur = s_par[t];
    while (cur >= 0) {
      const float* ki = s_kq + cur * KQ_LD;
      float pk = 0.f, pq = 0.f;
      for (int e = lane; e < DK; e += kWave) {
        pk = fmaf(kt[e], ki[e], pk);
        pq = fmaf(qt[e], ki[e], pq);
      }
      pk = wave_sum(pk);
      pq = wave_sum(pq);
      if (lane == 0) {
        s_A[t * CO_LD + cur] = s_gb[t] * gprod * pk;
        s_O[t * CO_LD + cur] = gprod * pq;
      }
      gprod *= s_ga[cur];
      cur = s_par[cur];
    }
    if (lane == 0) {
      s_O[t * CO_LD + t] = qk_self;
      s_gam[t] = gprod;
    }
  }

  // (6) [K;Q] S0^T on fp32 MFMA (16x16x4), A from LDS, B from registers.
  floatx4 acc[TPW][NRB];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) acc[tt][rb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int sec0 = (rb * 16) % TMAX;  // first node index of this 16-row block
    if (TMAX >= 16 && sec0 >= T) continue;
#pragma unroll
    for (int m = 0; m < MSTEPS; ++m) {
      const floatx4 av = *reinterpret_cast<const floatx4*>(s_kq + (rb * 16 + c16) * KQ_LD + 16 * m + 4 * kk);
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        if (wave + tt * NWAVE < NTILE) {
          acc[tt][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], sreg[tt][m][0], acc[tt][rb], 0, 0, 0);
          acc[tt][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[1], sreg[tt][m][1], acc[tt][rb], 0, 0, 0);
          acc[tt][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[2], sreg[tt][m][2], acc[tt][rb], 0, 0, 0);
          acc[tt][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[3], sreg[tt][m][3], acc[tt][rb], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();  // all reads of k/q done before W/Z overwrite the region

  float* s_wz = s_kq;  // [KQ_ROWS][WZ_LD]: rows [0,TMAX) = W = K S0^T, then Z = Q S0^T
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int tile = wave + tt * NWAVE;
    if (tile < NTILE) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s_wz[(rb * 16 + 4 * kk + r) * WZ_LD + tile * 16 + c16] = acc[tt][rb][r];
    }
  }
  __syncthreads();

  // (7) Per row of S: v by conv, forward substitution for u, then o.
  if (tid < ROWS) {
    const int i = r0 + tid;
    const int ch = 2 * p.Hk * DK + hv * DV + i;
    float w[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      w[j] = j < K ? p.conv_w[(static_cast<size_t>(l) * p.C + ch) * K + j] : 0.f;
    for (int t = 0; t < T; ++t) {
      const float vt = conv_at(p, x, cs, s_widx + t * kMaxK, w, K, lb, ch);
      float u = s_gb[t] * (vt - s_gam[t] * s_wz[t * WZ_LD + tid]);
      const unsigned long long anc = s_anc[t];
      for (unsigned long long m = anc; m; m &= m - 1) {
        const int a = __builtin_ctzll(m);
        u = fmaf(-s_A[t * CO_LD + a], s_wz[a * WZ_LD + tid], u);
      }
      s_wz[t * WZ_LD + tid] = u;  // W[t] -> U[t]; only this thread touches the column
      float o = fmaf(s_gam[t], s_wz[(TMAX + t) * WZ_LD + tid], s_O[t * CO_LD + t] * u);
      for (unsigned long long m = anc; m; m &= m - 1) {
        const int a = __builtin_ctzll(m);
        o = fmaf(s_O[t * CO_LD + a], s_wz[a * WZ_LD + tid], o);
      }
      const size_t oi = ((lb * T + t) * p.Hv + hv) * DV + i;
      p.o[oi] = o;
      p.tu[oi] = u;
    }
  }
}

template <int DK, int DV, typename TIn>
hipError_t launch_t(const VerifyArgs& a, hipStream_t s) {
  constexpr int ROWS = DV >= 64 ? 64 : DV;
  const int nsub = (a.Hv / a.Hk) * (DV / ROWS);
  const int n_units = a.L * a.B * a.Hk;
  const int grid = ((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * nsub;
  if (a.T <= 8)
    hipLaunchKernelGGL((k_verify_wy<DK, DV, 8, ROWS, TIn>), dim3(grid), dim3(256), 0, s, a);
  else if (a.T <= 16)
    hipLaunchKernelGGL((k_verify_wy<DK, DV, 16, ROWS, TIn>), dim3(grid), dim3(256), 0, s, a);
  else if (a.T <= 32)
    hipLaunchKernelGGL((k_verify_wy<DK, DV, 32, ROWS, TIn>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_verify_wy<DK, DV, 64, ROWS, TIn>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_d(const VerifyArgs& a, int dk, int dv, hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 32: return launch_t<32, 32, TIn>(a, s);
    case 64: return launch_t<64, 64, TIn>(a, s);
    case 128: return launch_t<128, 128, TIn>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_verify_wy(const VerifyArgs& a, int dk, int dv, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_d<uint16_t>(a, dk, dv, s) : launch_d<float>(a, dk, dv, s);
}

}  // namespace gdn
