// k_verify_wy.hip -- chunked (WY / UT-transform) verify of a draft chain or
// draft tree through one GDN layer, for gfx950.
//
// The gated delta rule (GDN page s2.1; replay form in s4), per node t with
// parent p (chain: p = t-1; -1 = the committed state S0):
//   S_t = a_t S_p + u_t k_t^T,  u_t = b_t (v_t - a_t S_p k_t),  o_t = S_t q_t.
// Unrolled along each node's ancestor path (Gamma = products of a along it):
//   gamma_t = prod of a over t and its ancestors,  Gamma[t,i] = gamma_t / gamma_i
//   (I + A) U = RHS,   A[t,i] = b_t Gamma[t,i] k_t.k_i  (i a proper ancestor of t)
//                      RHS_t  = b_t (v_t - gamma_t S0 k_t)
//   o_t = gamma_t S0 q_t + sum_{i in anc(t)+t} Oc[t,i] u_i,  Oc[t,i] = Gamma[t,i] q_t.k_i
// With Ti = (I + A)^-1 and M2 = Oc Ti (both T x T, supported on ancestors):
//   U = Ti RHS,   O = diag(gamma) Q S0^T + M2 RHS.
// The state enters only through [K;Q] S0^T, one dense (2T x Dk) x (Dk x Dv)
// contraction per head on fp32 MFMA with S0 read once from HBM into the
// B-operand registers; [Ti;M2] RHS is a second, small MFMA whose output lands
// in the same lanes as Q S0^T, so o and u leave straight from registers.  A
// tree is the same algebra with the ancestor set from the parent array
// (tree-aware verify, GDN page s8).  S0 and the conv window are never
// written: they stay the pre-verify snapshot that rollback replays onto.
//
// Work decomposition: one 256-thread workgroup per (layer, seq, v-head,
// ROWS-row block of S); the rows of S are independent recurrences sharing
// q, k and the gates.  Each wave owns 16-row tiles of S; lane (c16 = lane%16,
// kk = lane/16) holds S0[row c16][16m + 4kk .. +3] for every 16-column step m.

#include "gdn_common.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

constexpr int kMaxK = 8;
constexpr int kNT = 256;
constexpr int kNWave = kNT / kWave;

template <int DK, int DV, int TMAX, int ROWS, typename TIn>
struct VerifyLayout {
  static constexpr int KQ_ROWS = 2 * TMAX;  // k rows [0,TMAX), q rows [TMAX,2TMAX)
  static constexpr int KQ_LD = DK + 4;      // +4 floats: conflict-free float4 column reads
  static constexpr int RHS_LD = ROWS + 4;
  static constexpr int CO_LD = TMAX + 1;
  static constexpr int NCH = 2 * DK + ROWS;  // q, k of the k-head; v rows of the block
  static constexpr int XR = TMAX + kMaxK - 1;
  static constexpr int COEF_BYTES = 3 * TMAX * CO_LD * 4;
  static constexpr int STAGE_FULL = XR * NCH * (int)sizeof(TIn);
  static constexpr int STAGE_CAP = COEF_BYTES > 48 * 1024 ? COEF_BYTES : 48 * 1024;
  // channels staged per pass (multiple of 64 unless everything fits)
  static constexpr int CHK = STAGE_FULL <= STAGE_CAP
                                 ? NCH
                                 : ((STAGE_CAP / (XR * (int)sizeof(TIn))) / 64) * 64;
  static constexpr int STAGE_BYTES = XR * CHK * (int)sizeof(TIn);
  static constexpr int U1_BYTES = STAGE_BYTES > COEF_BYTES ? STAGE_BYTES : COEF_BYTES;
  static constexpr int KQ_BYTES = KQ_ROWS * KQ_LD * 4;
  static constexpr int RHS_BYTES = TMAX * RHS_LD * 4;
  static_assert(CHK >= 64, "staging chunk too small");
};

template <int DK, int DV, int TMAX, int ROWS, typename TIn>
__global__ __launch_bounds__(kNT) void k_verify_wy(VerifyArgs p) {
  using LY = VerifyLayout<DK, DV, TMAX, ROWS, TIn>;
  constexpr int KQ_LD = LY::KQ_LD, RHS_LD = LY::RHS_LD, CO_LD = LY::CO_LD;
  constexpr int NCH = LY::NCH, CHK = LY::CHK;
  constexpr int NRB = LY::KQ_ROWS / 16;
  constexpr int NTILE = ROWS / 16;
  constexpr int TPW = (NTILE + kNWave - 1) / kNWave;
  constexpr int MSTEPS = DK / 16;
  constexpr int NRBLK = DV / ROWS;
  static_assert(ROWS % 16 == 0 && DV % ROWS == 0 && TMAX % 8 == 0, "tiling");

  __shared__ __align__(16) float s_kq[LY::KQ_ROWS * KQ_LD];
  __shared__ __align__(16) float s_rhs[TMAX * RHS_LD];        // v, then RHS
  __shared__ __align__(16) unsigned char s_u1[LY::U1_BYTES];  // staging, then coefficients
  __shared__ float s_gam[TMAX], s_ga[TMAX], s_gb[TMAX];
  __shared__ unsigned long long s_anc[TMAX];
  __shared__ int s_par[TMAX];
  __shared__ int s_widx[TMAX * kMaxK];
  __shared__ int s_bad;
  TIn* s_x = reinterpret_cast<TIn*>(s_u1);                      // [XR][CHK]
  float* s_A = reinterpret_cast<float*>(s_u1);                  // [TMAX][CO_LD], later M2
  float* s_Oc = s_A + TMAX * CO_LD;
  float* s_Ti = s_Oc + TMAX * CO_LD;

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

  // (1) State loads first: their HBM latency overlaps everything up to MFMA.
  floatx4 sreg[TPW][MSTEPS];
  const float* S_head = p.S + (lb * p.Hv + hv) * static_cast<size_t>(DV * DK);
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int tile = wave + tt * kNWave;
    if (tile < NTILE) {
      const float* rp = S_head + static_cast<size_t>(r0 + tile * 16 + c16) * DK + 4 * kk;
#pragma unroll
      for (int m = 0; m < MSTEPS; ++m)
        sreg[tt][m] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(rp + 16 * m));
    }
  }

  // (2) Parents (validated) and gates.
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
    s_ga[tid] = ld_in(static_cast<const TIn*>(p.a), gi);
    s_gb[tid] = ld_in(static_cast<const TIn*>(p.b), gi);
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0 && p.dev_err) atomicOr(p.dev_err, GDN_DEV_ERR_PARENT);
    return;
  }
  if (tid < T) {
    if (rblk == 0) p.tg[(lb * T + tid) * p.Hv + hv] = s_ga[tid];
    // conv window of node tid: the node, its ancestors upward, then old rows
    int cur = tid, old = 0;
    for (int j = K - 1; j >= 0; --j) {
      if (cur >= 0) {
        s_widx[tid * kMaxK + j] = cur;
        cur = s_par[cur];
      } else {
        s_widx[tid * kMaxK + j] = --old;
      }
    }
    // gamma_t: product of a over the node and all its ancestors
    float gm = 1.f;
    for (int c = tid; c >= 0; c = s_par[c]) gm *= s_ga[c];
    s_gam[tid] = gm;
  }
  if (tid == 0) {
    for (int v = 0; v < T; ++v) {
      const int pv = s_par[v];
      s_anc[v] = pv < 0 ? 0ull : (s_anc[pv] | (1ull << pv));
    }
  }
  __syncthreads();
  if (p.conv_win && l == 0 && hk == 0 && g == 0 && rblk == 0) {
    for (int e = tid; e < T * K; e += kNT)
      p.conv_win[static_cast<size_t>(bb) * T * K + e] = s_widx[(e / K) * kMaxK + (e % K)];
  }

  // (3) Conv + SiLU of this block's q, k and v channels for every node:
  //     stage the raw rows [old window; x of all nodes] in LDS with one wide
  //     burst of independent loads, then convolve out of LDS.
  const TIn* x = static_cast<const TIn*>(p.x);
  const TIn* cs = static_cast<const TIn*>(p.conv_state);
  const int nrows = K - 1 + T;
  for (int c0 = 0; c0 < NCH; c0 += CHK) {
    const int nc = NCH - c0 < CHK ? NCH - c0 : CHK;
    for (int e = tid; e < nrows * nc; e += kNT) {
      const int row = e / nc, cl = e % nc, c = c0 + cl;
      const int ch = c < DK ? hk * DK + c
                            : (c < 2 * DK ? p.Hk * DK + hk * DK + (c - DK)
                                          : 2 * p.Hk * DK + hv * DV + r0 + (c - 2 * DK));
      s_x[row * CHK + cl] = row < K - 1 ? cs[(lb * (K - 1) + row) * p.C + ch]
                                        : x[(lb * T + (row - (K - 1))) * p.C + ch];
    }
    __syncthreads();
    for (int cl = tid; cl < nc; cl += kNT) {
      const int c = c0 + cl;
      const int ch = c < DK ? hk * DK + c
                            : (c < 2 * DK ? p.Hk * DK + hk * DK + (c - DK)
                                          : 2 * p.Hk * DK + hv * DV + r0 + (c - 2 * DK));
      float w[kMaxK];
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        w[j] = j < K ? p.conv_w[(static_cast<size_t>(l) * p.C + ch) * K + j] : 0.f;
      float* dst;
      int ld;
      if (c < DK) {
        dst = s_kq + TMAX * KQ_LD + c;
        ld = KQ_LD;
      } else if (c < 2 * DK) {
        dst = s_kq + (c - DK);
        ld = KQ_LD;
      } else {
        dst = s_rhs + (c - 2 * DK);
        ld = RHS_LD;
      }
      for (int t = 0; t < TMAX; ++t) {
        float y = 0.f;
        if (t < T) {
#pragma unroll
          for (int j = 0; j < kMaxK; ++j)
            if (j < K)
              y = fmaf(w[j], ld_in(s_x, (s_widx[t * kMaxK + j] + K - 1) * CHK + cl), y);
          if (p.silu) y = y / (1.f + __expf(-y));
        }
        dst[t * ld] = y;
      }
    }
    __syncthreads();
  }

  // (4) L2-normalise the 2T vectors (k rows then q rows), one wave per vector.
  for (int vi = wave; vi < 2 * T; vi += kNWave) {
    float* r = s_kq + (vi < T ? vi : TMAX + vi - T) * KQ_LD;
    float ss = 0.f;
    for (int e = lane; e < DK; e += kWave) ss = fmaf(r[e], r[e], ss);
    ss = wave_sum(ss);
    const float inv = 1.f / sqrtf(ss + p.eps);
    for (int e = lane; e < DK; e += kWave) r[e] *= inv;
  }
  __syncthreads();

  // Tape k: written once per k-head (first v-head of the group, first row block).
  if (g == 0 && rblk == 0) {
    for (int e = tid; e < T * DK; e += kNT) {
      const int t = e / DK, c = e % DK;
      p.tk[((lb * T + t) * p.Hk + hk) * DK + c] = s_kq[t * KQ_LD + c];
    }
  }

  // (5) Coefficients A (proper ancestors) and Oc (ancestors + self), dense
  //     TMAX x TMAX with zeros elsewhere; one thread per (t, i) pair.
  for (int e = tid; e < TMAX * TMAX; e += kNT) {
    const int t = e / TMAX, i = e % TMAX;
    float av = 0.f, ov = 0.f;
    if (t < T && i <= t && (i == t || ((s_anc[t] >> i) & 1ull))) {
      float gm = 1.f;  // Gamma[t,i]: product of a from t up to, not including, i
      for (int c = t; c != i; c = s_par[c]) gm *= s_ga[c];
      const floatx4* kt = reinterpret_cast<const floatx4*>(s_kq + t * KQ_LD);
      const floatx4* ki = reinterpret_cast<const floatx4*>(s_kq + i * KQ_LD);
      const floatx4* qt = reinterpret_cast<const floatx4*>(s_kq + (TMAX + t) * KQ_LD);
      floatx4 dk = {0.f, 0.f, 0.f, 0.f}, dq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
      for (int c = 0; c < DK / 4; ++c) {
        const floatx4 kiv = ki[c];
        const floatx4 ktv = kt[c];
        const floatx4 qtv = qt[c];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          dk[h] = fmaf(ktv[h], kiv[h], dk[h]);
          dq[h] = fmaf(qtv[h], kiv[h], dq[h]);
        }
      }
      const float kdot = (dk[0] + dk[1]) + (dk[2] + dk[3]);
      const float qdot = (dq[0] + dq[1]) + (dq[2] + dq[3]);
      av = i == t ? 0.f : s_gb[t] * gm * kdot;
      ov = gm * qdot;
    }
    s_A[t * CO_LD + i] = av;
    s_Oc[t * CO_LD + i] = ov;
  }

  // (6) [K;Q] S0^T on fp32 MFMA (16x16x4): A from LDS, B from registers.
  floatx4 acc1[TPW][NRB];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) acc1[tt][rb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    if (TMAX >= 16 && (rb * 16) % TMAX >= T) continue;  // all-padding block
#pragma unroll
    for (int m = 0; m < MSTEPS; ++m) {
      const floatx4 av =
          *reinterpret_cast<const floatx4*>(s_kq + (rb * 16 + c16) * KQ_LD + 16 * m + 4 * kk);
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        if (wave + tt * kNWave < NTILE) {
#pragma unroll
          for (int h = 0; h < 4; ++h)
            acc1[tt][rb] =
                __builtin_amdgcn_mfma_f32_16x16x4f32(av[h], sreg[tt][m][h], acc1[tt][rb], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();  // A and Oc complete

  // (7) Ti = (I + A)^-1, one thread per column j (forward substitution).
  if (tid < TMAX) {
    const int j = tid;
    for (int t = 0; t < TMAX; ++t) {
      float xv = 0.f;
      if (t < T && j < T) {
        if (t == j) {
          xv = 1.f;
        } else if (t > j) {
          const unsigned long long m = s_anc[t] & ~((1ull << j) - 1ull);
          for (unsigned long long mm = m; mm; mm &= mm - 1) {
            const int a = __builtin_ctzll(mm);
            xv = fmaf(-s_A[t * CO_LD + a], s_Ti[a * CO_LD + j], xv);
          }
        }
      }
      s_Ti[t * CO_LD + j] = xv;
    }
  }
  // RHS_t[i] = b_t (v_t[i] - gamma_t W[t][i]) from the W rows of acc1, in place
  // of v in s_rhs; padding rows become 0.
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int tile = wave + tt * kNWave;
    if (tile < NTILE) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rb * 16 + 4 * kk + r;
          if (row < TMAX) {
            float* d = s_rhs + row * RHS_LD + tile * 16 + c16;
            *d = row < T ? s_gb[row] * (*d - s_gam[row] * acc1[tt][rb][r]) : 0.f;
          }
        }
      }
    }
  }
  __syncthreads();  // Ti and RHS complete

  // (8) M2 = Oc Ti (support: ancestors-or-self), written over A.
  for (int e = tid; e < TMAX * TMAX; e += kNT) {
    const int t = e / TMAX, s = e % TMAX;
    float mv = 0.f;
    if (t < T && s <= t) {
      mv = s_Oc[t * CO_LD + t] * s_Ti[t * CO_LD + s];
      const unsigned long long m = s_anc[t] & ~((1ull << s) - 1ull);
      for (unsigned long long mm = m; mm; mm &= mm - 1) {
        const int a = __builtin_ctzll(mm);
        mv = fmaf(s_Oc[t * CO_LD + a], s_Ti[a * CO_LD + s], mv);
      }
    }
    s_A[t * CO_LD + s] = mv;
  }
  __syncthreads();

  // (9) [Ti; M2] RHS on MFMA: rows [0,TMAX) give U, rows [TMAX,2TMAX) give
  //     M2 RHS, in the same lanes as the Q S0^T rows of acc1.
  floatx4 acc2[TPW][NRB];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) acc2[tt][rb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    if (TMAX >= 16 && (rb * 16) % TMAX >= T) continue;
    const int arow = rb * 16 + c16;
    const float* amat = arow < TMAX ? s_Ti + arow * CO_LD : s_A + (arow - TMAX) * CO_LD;
#pragma unroll
    for (int st = 0; st < TMAX / 4; ++st) {
      if (st * 4 >= T) break;
      const float a_op = amat[4 * st + kk];
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const int tile = wave + tt * kNWave;
        if (tile < NTILE) {
          const float b_op = s_rhs[(4 * st + kk) * RHS_LD + tile * 16 + c16];
          acc2[tt][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_op, b_op, acc2[tt][rb], 0, 0, 0);
        }
      }
    }
  }

  // (10) Outputs straight from registers: u rows and o = gamma Z + M2 RHS.
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int tile = wave + tt * kNWave;
    if (tile < NTILE) {
      const int i = r0 + tile * 16 + c16;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rb * 16 + 4 * kk + r;
          const int t = row < TMAX ? row : row - TMAX;
          if (t < T) {
            const size_t oi = ((lb * T + t) * p.Hv + hv) * DV + i;
            if (row < TMAX)
              p.tu[oi] = acc2[tt][rb][r];
            else
              p.o[oi] = fmaf(s_gam[t], acc1[tt][rb][r], acc2[tt][rb][r]);
          }
        }
      }
    }
  }
}

template <int DK, int DV, int ROWS, typename TIn>
hipError_t launch_t(const VerifyArgs& a, hipStream_t s) {
  const int nsub = (a.Hv / a.Hk) * (DV / ROWS);
  const int n_units = a.L * a.B * a.Hk;
  const long long grid = static_cast<long long>((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * nsub;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.T <= 8)
    hipLaunchKernelGGL((k_verify_wy<DK, DV, 8, ROWS, TIn>), dim3(grid), dim3(kNT), 0, s, a);
  else if (a.T <= 16)
    hipLaunchKernelGGL((k_verify_wy<DK, DV, 16, ROWS, TIn>), dim3(grid), dim3(kNT), 0, s, a);
  else if (a.T <= 32)
    hipLaunchKernelGGL((k_verify_wy<DK, DV, 32, ROWS, TIn>), dim3(grid), dim3(kNT), 0, s, a);
  else
    hipLaunchKernelGGL((k_verify_wy<DK, DV, 64, ROWS, TIn>), dim3(grid), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_d(const VerifyArgs& a, int dk, int dv, hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 32: return launch_t<32, 32, 32, TIn>(a, s);
    case 64: return launch_t<64, 64, 64, TIn>(a, s);
    case 128: return launch_t<128, 128, 64, TIn>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_verify_wy(const VerifyArgs& a, int dk, int dv, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_d<uint16_t>(a, dk, dv, s) : launch_d<float>(a, dk, dv, s);
}

}  // namespace gdn
