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
// The state enters only through S0 [K;Q]^T, one dense (Dv x Dk) x (Dk x 2T)
// contraction per head on bf16 MFMA with hi/lo operand splits (fp32-level
// accuracy), S0 read once from HBM straight into the A-operand registers;
// RHS^T [Ti;M2]^T is a second, small MFMA whose output lands in the same
// lanes as S0 Q^T, so o and u leave straight from registers.  A tree is the
// same algebra with the ancestor set from the parent array (tree-aware
// verify, GDN page s8).  S0 and the conv window are never written: they stay
// the pre-verify snapshot that rollback replays onto.
//
// Work decomposition: one workgroup per (layer, seq, v-head, ROWS-row block
// of S); the rows of S are independent recurrences sharing q, k and the
// gates.  Each wave owns 16-row tiles of S; lane (c16 = lane%16, kk =
// lane/16) holds S0[row c16][16m + 4kk .. +3] for every 16-column step m.
// The per-head prologue (conv, L2 norm, Gram on MFMA, the T x T algebra)
// runs while the state loads are in flight.

#include "gdn_common.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

constexpr int kMaxK = 8;

// Threads per workgroup: eight waves for 64-node chunks (one workgroup per CU
// by LDS, so its latency-bound phases get more lanes), four waves otherwise.
template <int TMAX>
constexpr int threads_for() {
  return TMAX >= 64 ? 512 : 256;
}

// Waves per SIMD to keep resident: chunks of up to 16 nodes fit four
// workgroups per CU in LDS, so registers must not be what limits them
// (at most 128 per lane); longer chunks are held to two or one by LDS.
template <int TMAX>
constexpr int waves_per_eu() {
  return TMAX <= 16 ? 4 : 1;
}

// Sum over aligned groups of 8 lanes (DPP; every lane gets its group's sum).
__device__ __forceinline__ float sum8(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ float silu(float y) {
  return y * __builtin_amdgcn_rcpf(1.f + __expf(-y));
}

// Back to the input dtype; exact for values that were widened from it.
template <typename TIn>
__device__ __forceinline__ TIn to_in(float v);
template <>
__device__ __forceinline__ float to_in<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t to_in<uint16_t>(float v) {
  return static_cast<uint16_t>(__float_as_uint(v) >> 16);
}

template <int DK, int DV, int TMAX, int ROWS, int KM, typename TIn>
struct VerifyLayout {
  static constexpr int KQ_ROWS = 2 * TMAX;  // k rows [0,TMAX), q rows [TMAX,2TMAX)
  static constexpr int KQ_LD = DK + 4;      // +4 floats: conflict-free float4 column reads
  // RHS stored transposed, [ROWS][RT_LD]: odd stride (conflict-free scalar
  // access) for short chunks, multiple of 4 (float4 access) for long ones.
  static constexpr int RT_LD = TMAX <= 16 ? TMAX + 1 : TMAX + 4;
  static constexpr int CO_LD = TMAX + 4;  // multiple of 4: float4 row reads
  static constexpr int NCH = 2 * DK + ROWS;  // q, k of the k-head; v rows of the block
  static constexpr int XR = TMAX + KM - 1;
  // Raw conv inputs [old window rows; node rows] x [q | k | v-rows], staged
  // with 16-byte loads; CPR = 16-byte chunks per row.
  static constexpr int CPR = NCH * (int)sizeof(TIn) / 16;
  static constexpr int STAGE_BYTES = XR * CPR * 16;
  static constexpr int COEF_BYTES = 3 * TMAX * CO_LD * 4;  // [A;Oc] then [M2;Oc], and Ti
  static constexpr int U1_BYTES = STAGE_BYTES > COEF_BYTES ? STAGE_BYTES : COEF_BYTES;
  static constexpr int TOTAL = 2 * TMAX * KQ_LD * 4 + ROWS * RT_LD * 4 + U1_BYTES + TMAX * (24 + 4 * KM) + 16;
  static_assert(TOTAL <= 160 * 1024, "LDS budget of one workgroup exceeded");
};

template <int DK, int DV, int TMAX, int ROWS, int KC, typename TIn>
__global__ __launch_bounds__(threads_for<TMAX>())
__attribute__((amdgpu_waves_per_eu(waves_per_eu<TMAX>()))) void k_verify_wy(VerifyArgs p) {
  constexpr int kNT = threads_for<TMAX>();
  constexpr int kNWave = kNT / kWave;
  constexpr int KM = KC > 0 ? KC : kMaxK;  // unroll bound of the conv taps
  static_assert(KM == 4 || KM == 8, "window rows are read as int4");
  using LY = VerifyLayout<DK, DV, TMAX, ROWS, KM, TIn>;
  constexpr int KQ_LD = LY::KQ_LD, RT_LD = LY::RT_LD, CO_LD = LY::CO_LD;
  constexpr int NCH = LY::NCH;
  constexpr int NRB = LY::KQ_ROWS / 16;
  constexpr int NTILE = ROWS / 16;
  constexpr int TPW = (NTILE + kNWave - 1) / kNWave;
  constexpr int MSTEPS = DK / 16;
  constexpr int NRBLK = DV / ROWS;
  static_assert(ROWS % 16 == 0 && DV % ROWS == 0 && TMAX % 8 == 0 && TMAX <= 64, "tiling");

  __shared__ __align__(16) float s_kq[LY::KQ_ROWS * KQ_LD];
  __shared__ __align__(16) float s_rhs[ROWS * RT_LD];         // v, then RHS, [row of S][node]
  __shared__ __align__(16) unsigned char s_u1[LY::U1_BYTES];  // staging, then coefficients
  __shared__ float s_gam[TMAX], s_ga[TMAX], s_gb[TMAX];
  __shared__ unsigned long long s_anc[TMAX];
  __shared__ int s_par[TMAX];
  __shared__ __align__(16) int s_widx[TMAX * KM];  // conv window rows per node
  __shared__ int s_bad;
  float* s_G = reinterpret_cast<float*>(s_u1);  // [2TMAX][CO_LD]: KK then A (-> M2); QK then Oc
  float* s_Ti = s_G + 2 * TMAX * CO_LD;         // [TMAX][CO_LD]

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
  const int K = KC > 0 ? KC : p.K;
  const bool tree = p.parent != nullptr;

  // (1) Issue the small loads, then the first group of state loads.
  //     Vector-memory loads return in order, so the prologue below waits only
  //     for the small loads while the state stays in flight.
  const TIn* x = static_cast<const TIn*>(p.x);
  const TIn* cs = static_cast<const TIn*>(p.conv_state);
  const float* cw = p.conv_w + static_cast<size_t>(l) * p.C * K;
  const TIn* xcol = x + lb * T * p.C;
  const TIn* ccol = cs + lb * (K - 1) * p.C;
  auto chan = [&](int c) {
    return c < DK ? hk * DK + c
                  : (c < 2 * DK ? p.Hk * DK + hk * DK + (c - DK)
                                : 2 * p.Hk * DK + hv * DV + r0 + (c - 2 * DK));
  };
  // Every load below is unconditional, from a clamped always-valid address,
  // with the value selected afterwards: a load under a branch makes the
  // compiler wait for it at the join, which would serialise the prologue.
  const int tq = tid < T ? tid : 0;
  const int* par_ptr = tree ? p.parent + static_cast<size_t>(bb) * T + tq
                            : reinterpret_cast<const int*>(p.S);
  const int par_raw = *par_ptr;
  const size_t gi = (lb * T + tq) * p.Hv + hv;
  const float ga_ld = ld_in(static_cast<const TIn*>(p.a), gi);
  const float gb_ld = ld_in(static_cast<const TIn*>(p.b), gi);
  // Raw conv inputs: rows [old window; nodes] x channels [q | k | v-rows],
  // each row three contiguous segments, fetched as 16-byte chunks.
  constexpr int CPR = LY::CPR;
  constexpr int EPC = 16 / (int)sizeof(TIn);  // elements per chunk
  constexpr int XRR = TMAX + KM - 1;
  constexpr int NRAW = (XRR * CPR + kNT - 1) / kNT;
  const int nrows = K - 1 + T;
  u32x4 raw[NRAW];
#pragma unroll
  for (int q = 0; q < NRAW; ++q) {
    const int e = tid + q * kNT;
    const int row = e / CPR, chunk = e % CPR;
    const int rr = row < nrows ? row : nrows - 1;
    const int c = chunk * EPC;  // first channel of the chunk
    const TIn* base = rr < K - 1 ? ccol + static_cast<size_t>(rr) * p.C
                                 : xcol + static_cast<size_t>(rr - (K - 1)) * p.C;
    raw[q] = *reinterpret_cast<const u32x4*>(base + chan(c));
  }
  // conv weights of this thread's channels (one float4 when K == 4)
  constexpr int NSLOT = (NCH + kNT - 1) / kNT;
  float w[NSLOT][KM];
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) {
    const int c = tid + sl * kNT;
    const bool live = c < NCH;
    const int ch = chan(live ? c : 0);
    if (KC == 4) {
      const floatx4 wv = *reinterpret_cast<const floatx4*>(cw + static_cast<size_t>(ch) * 4);
#pragma unroll
      for (int j = 0; j < KM; ++j) w[sl][j] = live ? wv[j] : 0.f;
    } else {
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        const int jj = j < K ? j : 0;
        const float wv = cw[static_cast<size_t>(ch) * K + jj];
        w[sl][j] = (live && j < K) ? wv : 0.f;
      }
    }
  }
  // The state loads are unconditional too (a wave without a tile re-reads
  // the last one): with loads under a branch the compiler can only count the
  // loads issued on every path, and the first use of a small input would
  // then wait for the whole state to arrive.  They go out in four groups
  // between the prologue phases: a wave cannot issue past a load the memory
  // pipeline has no room for, so issuing all 16 KiB at once would hold the
  // prologue until most of the CU's state had arrived; in groups the queue
  // stays full while the phases run in between.
  floatx4 sreg[TPW][MSTEPS];
  const float* S_head = p.S + (lb * p.Hv + hv) * static_cast<size_t>(DV * DK);
  auto load_state = [&](int grp) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int tile = wave + tt * kNWave < NTILE ? wave + tt * kNWave : NTILE - 1;
      const float* rp = S_head + static_cast<size_t>(r0 + tile * 16 + c16) * DK + 4 * kk;
#pragma unroll
      for (int m = 0; m < MSTEPS; ++m)
        if (m * 4 / MSTEPS == grp) sreg[tt][m] = *reinterpret_cast<const floatx4*>(rp + 16 * m);
    }
  };
  load_state(0);

  // (2) Parents (validated) and gates.
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (tid < T) {
    int pv = tree ? par_raw : tid - 1;
    if (pv < -1 || pv >= tid) {
      s_bad = 1;
      pv = -1;
    }
    s_par[tid] = pv;
    s_ga[tid] = ga_ld;
    s_gb[tid] = gb_ld;
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0 && p.dev_err) atomicOr(p.dev_err, GDN_DEV_ERR_PARENT);
    return;
  }
  if (tid >= T && tid < TMAX) {  // padding nodes read a valid (discarded) window
#pragma unroll
    for (int j = 0; j < KM; ++j) s_widx[tid * KM + j] = 0;
  }
  if (tid < T) {
    if (rblk == 0) p.tg[(lb * T + tid) * p.Hv + hv] = s_ga[tid];
    // slots beyond the kernel width stay valid row indices (the conv reads
    // every slot; their weights are zero)
    for (int j = K; j < KM; ++j) s_widx[tid * KM + j] = 0;
    // conv window of node tid: the node, its ancestors upward, then old rows
    int cur = tid, old = 0;
    for (int j = K - 1; j >= 0; --j) {
      if (cur >= 0) {
        s_widx[tid * KM + j] = cur;
        cur = s_par[cur];
      } else {
        s_widx[tid * KM + j] = --old;
      }
    }
  }
  if (tid < T) {  // proper-ancestor bitmask of node tid
    unsigned long long m = 0ull;
    if (tree) {
      for (int c = s_par[tid]; c >= 0; c = s_par[c]) m |= 1ull << c;
    } else {
      m = tid == 0 ? 0ull : (~0ull >> (64 - tid));
    }
    s_anc[tid] = m;
  }
  __syncthreads();
  if (p.conv_win && l == 0 && hk == 0 && g == 0 && rblk == 0) {
    for (int e = tid; e < T * K; e += kNT)
      p.conv_win[static_cast<size_t>(bb) * T * K + e] = s_widx[(e / K) * KM + (e % K)];
  }

  // (3) Conv + SiLU out of the staged raw block, one thread per channel.
  u32x4* s_raw = reinterpret_cast<u32x4*>(s_u1);  // [XRR][CPR]
#pragma unroll
  for (int q = 0; q < NRAW; ++q) {
    const int e = tid + q * kNT;
    if (e < nrows * CPR) s_raw[e] = raw[q];
  }
  __syncthreads();
  const TIn* s_rawe = reinterpret_cast<const TIn*>(s_u1);  // element view [XRR][NCH]
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) {
    const int c = tid + sl * kNT;
    if (c < NCH) {
      float* dst;
      int ld;
      if (c < DK) {
        dst = s_kq + TMAX * KQ_LD + c;
        ld = KQ_LD;
      } else if (c < 2 * DK) {
        dst = s_kq + (c - DK);
        ld = KQ_LD;
      } else {
        dst = s_rhs + (c - 2 * DK) * RT_LD;
        ld = 1;
      }
      // Branch-free over nodes: padding nodes read valid rows and are zeroed.
      // Each batch reads all of its inputs before its first store, so the
      // LDS reads of a batch are in flight together instead of one round
      // trip per node behind the previous node's store.
      if (!tree) {
        // chain: the window of token t is raw rows t .. t+K-1
        constexpr int CH = 8;
#pragma unroll
        for (int t0 = 0; t0 < TMAX; t0 += CH) {
          float xr[CH + KM - 1];
#pragma unroll
          for (int j = 0; j < CH + KM - 1; ++j) xr[j] = ld_in(s_rawe, (t0 + j) * NCH + c);
#pragma unroll
          for (int tt = 0; tt < CH; ++tt) {
            float y = 0.f;
#pragma unroll
            for (int j = 0; j < KM; ++j)
              if (KC > 0 || j < K) y = fmaf(w[sl][j], xr[tt + j], y);
            if (p.silu) y = silu(y);
            dst[(t0 + tt) * ld] = t0 + tt < T ? y : 0.f;
          }
        }
      } else {
        constexpr int NB = TMAX <= 16 ? 2 : 4;  // nodes per batch (registers: the state is live)
#pragma unroll
        for (int t0 = 0; t0 < TMAX; t0 += NB) {
          int wi[NB][KM];
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            const int4 wa = *reinterpret_cast<const int4*>(s_widx + (t0 + n) * KM);
            wi[n][0] = wa.x;
            if (KM > 1) wi[n][1 % KM] = wa.y;
            if (KM > 2) wi[n][2 % KM] = wa.z;
            if (KM > 3) wi[n][3 % KM] = wa.w;
            if constexpr (KM > 4) {
              const int4 wb = *reinterpret_cast<const int4*>(s_widx + (t0 + n) * KM + 4);
              wi[n][4 % KM] = wb.x;
              wi[n][5 % KM] = wb.y;
              wi[n][6 % KM] = wb.z;
              wi[n][7 % KM] = wb.w;
            }
          }
          float xv[NB][KM];
#pragma unroll
          for (int n = 0; n < NB; ++n)
#pragma unroll
            for (int j = 0; j < KM; ++j) xv[n][j] = ld_in(s_rawe, (wi[n][j] + K - 1) * NCH + c);
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            float y = 0.f;
#pragma unroll
            for (int j = 0; j < KM; ++j)
              if (KC > 0 || j < K) y = fmaf(w[sl][j], xv[n][j], y);
            if (p.silu) y = silu(y);
            dst[(t0 + n) * ld] = t0 + n < T ? y : 0.f;
          }
        }
      }
    }
  }
  __syncthreads();

  load_state(1);

  // (4) L2-normalise the 2T vectors (k rows, q rows): 8 lanes per vector.
  for (int v0 = 0; v0 < 2 * T; v0 += kNT / 8) {
    const int vi = v0 + tid / 8, sub = tid % 8;
    const bool ok = vi < 2 * T;
    floatx4* r = reinterpret_cast<floatx4*>(s_kq + (vi < T ? vi : TMAX + vi - T) * KQ_LD);
    floatx4 e[DK / 32];
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < DK / 32; ++q) {
      e[q] = ok ? r[sub + 8 * q] : floatx4{0.f, 0.f, 0.f, 0.f};
      ss = fmaf(e[q][0], e[q][0], fmaf(e[q][1], e[q][1], fmaf(e[q][2], e[q][2], fmaf(e[q][3], e[q][3], ss))));
    }
    ss = sum8(ss);
    const float inv = 1.f / sqrtf(ss + p.eps);
    if (ok) {
#pragma unroll
      for (int q = 0; q < DK / 32; ++q) r[sub + 8 * q] = e[q] * inv;
    }
  }
  __syncthreads();

  // Tape k: written once per k-head (first v-head of the group, first row block).
  if (g == 0 && rblk == 0) {
    for (int e = tid; e < T * (DK / 4); e += kNT) {
      const int t = e / (DK / 4), c4 = e % (DK / 4);
      __builtin_nontemporal_store(reinterpret_cast<const floatx4*>(s_kq + t * KQ_LD)[c4],
                                  reinterpret_cast<floatx4*>(p.tk + ((lb * T + t) * p.Hk + hk) * DK) + c4);
    }
  }

  // (5) Gram [K;Q] K^T on bf16x3 MFMA: G[r][i] = (k or q)_r . k_i.
  {
    constexpr int NCT = (TMAX + 15) / 16;
    for (int job = wave; job < NRB * NCT; job += kNWave) {
      const int rb = job / NCT, ct = job % NCT;
      const bool live = !(TMAX >= 16 && (rb * 16) % TMAX >= T) && ct * 16 < T;
      if (!live) continue;
      floatx4 gacc = {0.f, 0.f, 0.f, 0.f};
      const float* arow = s_kq + (rb * 16 + c16) * KQ_LD + 4 * kk;
      const float* brow = s_kq + (ct * 16 + c16) * KQ_LD + 4 * kk;
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        bf16x8 ahi, alo, bhi, blo;
        split_bf16x8(*reinterpret_cast<const floatx4*>(arow + 32 * ks),
                     *reinterpret_cast<const floatx4*>(arow + 32 * ks + 16), ahi, alo);
        split_bf16x8(*reinterpret_cast<const floatx4*>(brow + 32 * ks),
                     *reinterpret_cast<const floatx4*>(brow + 32 * ks + 16), bhi, blo);
        gacc = mfma_bf16x3(ahi, alo, bhi, blo, gacc);
      }
      const int col = ct * 16 + c16;
      if (col < TMAX) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s_G[(rb * 16 + 4 * kk + r) * CO_LD + col] = gacc[r];
      }
    }
  }
  __syncthreads();

  load_state(2);

  // (6) gamma per node (walk to the root), then A and Oc in place of the
  //     Gram rows, one thread per (t, i): Gamma[t,i] = gamma_t / gamma_i, or
  //     the product of a along the path when gamma_i has underflowed.
  if (tid < T) {
    float gm = 1.f;
    if (!tree) {  // chain: independent reads, same product order as the walk
#pragma unroll
      for (int c = TMAX - 1; c >= 0; --c) gm *= c <= tid ? s_ga[c] : 1.f;
    } else {
      for (int c = tid; c >= 0; c = s_par[c]) gm *= s_ga[c];
    }
    s_gam[tid] = gm;
  }
  __syncthreads();
  // All reads of a thread's pairs come before its first store.
  constexpr int NPQ = (TMAX * TMAX + kNT - 1) / kNT;  // pairs per thread
  {
    float av[NPQ], ov[NPQ];
#pragma unroll
    for (int q = 0; q < NPQ; ++q) {
      const int e = tid + q * kNT;
      const int t = (e / TMAX) % TMAX, i = e % TMAX;
      const bool on = e < TMAX * TMAX && t < T && (i == t || ((s_anc[t] >> i) & 1ull));
      const float gi = s_gam[i], gt = s_gam[t], bt = s_gb[t];
      const float gk = s_G[t * CO_LD + i], gq = s_G[(TMAX + t) * CO_LD + i];
      float gm = gt / gi;
      if (on && !(gi > 1e-30f)) {  // gamma_i underflowed: product along the path
        gm = 1.f;
        for (int c = t; c != i; c = s_par[c]) gm *= s_ga[c];
      }
      av[q] = on && i != t ? bt * gm * gk : 0.f;
      ov[q] = on ? gm * gq : 0.f;
    }
#pragma unroll
    for (int q = 0; q < NPQ; ++q) {
      const int e = tid + q * kNT;
      if (e < TMAX * TMAX) {
        const int t = e / TMAX, i = e % TMAX;
        s_G[t * CO_LD + i] = av[q];
        s_G[(TMAX + t) * CO_LD + i] = ov[q];
      }
    }
  }
  __syncthreads();  // A, Oc, gamma complete

  // (7) Ti = (I + A)^-1 by columns (forward substitution, thread j = column).
  if (tid < TMAX) {
    const int j = tid;
    if (TMAX <= 16) {
      // column j by forward substitution; the column is stored only after
      // the solve, so every read of A can be in flight at once
      float xc[TMAX];
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        float v = (t == j) ? 1.f : 0.f;
#pragma unroll
        for (int a = 0; a < t; ++a) v = fmaf(-s_G[t * CO_LD + a], xc[a], v);
        xc[t] = (t < T && j < T) ? v : 0.f;
      }
#pragma unroll
      for (int t = 0; t < TMAX; ++t) s_Ti[t * CO_LD + j] = xc[t];
    }
  }
  if constexpr (TMAX > 16) {
    // Level by level over node depth: row t of Ti needs only rows of its
    // ancestors, which sit at smaller depths.  Thread pairs (t, s) fixed:
    // e = tid + q * kNT, with each pair's depth and ancestors in registers.
    constexpr int NQ = TMAX * TMAX / kNT;
    static_assert(TMAX * TMAX % kNT == 0, "pairs per thread");
    const int sc = tid % TMAX;
    int dq[NQ];
    unsigned long long aq[NQ];
    int md = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int t = (tid + q * kNT) / TMAX;
      aq[q] = t < T ? s_anc[t] : 0ull;
      dq[q] = t < T ? __popcll(aq[q]) : -1;
      md = dq[q] > md ? dq[q] : md;
      if (t >= T) s_Ti[t * CO_LD + sc] = 0.f;  // padding rows
    }
    if (tid == 0) s_bad = 0;
    __syncthreads();
    atomicMax(&s_bad, md);  // LDS max of depths (s_bad is free again)
    __syncthreads();
    md = s_bad;
    for (int d = 0; d <= md; ++d) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (dq[q] != d) continue;
        const int t = (tid + q * kNT) / TMAX;
        float v = 0.f;
        if (sc < T) {
          if (sc == t) {
            v = 1.f;
          } else if (sc < t) {
            for (unsigned long long mm = aq[q] & ~((1ull << sc) - 1ull); mm; mm &= mm - 1) {
              const int a = __builtin_ctzll(mm);
              v = fmaf(-s_G[t * CO_LD + a], s_Ti[a * CO_LD + sc], v);
            }
          }
        }
        s_Ti[t * CO_LD + sc] = v;
      }
      __syncthreads();
    }
  }
  __syncthreads();  // Ti complete

  load_state(3);

  // (8) M2 = Oc Ti (support: ancestors-or-self), written over A.
  if constexpr (TMAX <= 16) {
    for (int e = tid; e < TMAX * TMAX; e += kNT) {
      const int t = e / TMAX, sc = e % TMAX;
      float mv = 0.f;
      if (t < T && sc <= t) {
        const float* orow = s_G + (TMAX + t) * CO_LD;
        mv = orow[t] * s_Ti[t * CO_LD + sc];
        for (int a = sc; a < t; ++a) mv = fmaf(orow[a], s_Ti[a * CO_LD + sc], mv);
      }
      s_G[t * CO_LD + sc] = mv;
    }
  } else {
    // bf16x3 MFMA: A = Oc rows (float4 reads), B = Ti columns.
    constexpr int NB = TMAX / 16;
    for (int job = wave; job < NB * NB; job += kNWave) {
      const int rb = job / NB, ct = job % NB;
      floatx4 macc = {0.f, 0.f, 0.f, 0.f};
      const float* orow = s_G + (TMAX + rb * 16 + c16) * CO_LD + 8 * kk;
#pragma unroll
      for (int st = 0; st < TMAX / 32; ++st) {
        bf16x8 ahi, alo, bhi, blo;
        split_bf16x8(*reinterpret_cast<const floatx4*>(orow + 32 * st),
                     *reinterpret_cast<const floatx4*>(orow + 32 * st + 4), ahi, alo);
        floatx4 b0, b1;
        const float* tcol = s_Ti + (32 * st + 8 * kk) * CO_LD + ct * 16 + c16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          b0[e] = tcol[e * CO_LD];
          b1[e] = tcol[(e + 4) * CO_LD];
        }
        split_bf16x8(b0, b1, bhi, blo);
        macc = mfma_bf16x3(ahi, alo, bhi, blo, macc);
      }
      // the A rows are no longer read (Ti is complete): store the tile there
#pragma unroll
      for (int r = 0; r < 4; ++r) s_G[(rb * 16 + 4 * kk + r) * CO_LD + ct * 16 + c16] = macc[r];
    }
  }
  __syncthreads();

  // (9) S0 [K;Q]^T on bf16 MFMA (16x16x32) with every operand split into a
  //     bf16 high part and a bf16 residual (three products, fp32 accumulate).
  //     A = this wave's 16-row tile of S0 (from registers), B = a 16-column
  //     block of [K;Q] rows, so lane (n, kk) ends with rows i = 4kk..4kk+3 of
  //     the tile for one k or q row n: one node per lane, four consecutive
  //     state rows, which keeps the RHS in registers and the outputs float4.
  //     Step s contracts the 32 columns {32s + 16h + 4kk + e}: the two float4
  //     this lane holds for m = 2s, 2s+1, and the matching k/q columns.
  constexpr int KSTEPS = DK / 32;
  constexpr int NCB = NRB;  // 16-column blocks of [K;Q]: k rows, then q rows
  bf16x8 shi[TPW][KSTEPS], slo[TPW][KSTEPS];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      split_bf16x8(sreg[tt][2 * ks], sreg[tt][2 * ks + 1], shi[tt][ks], slo[tt][ks]);
  // this lane's node in each column block, its gates and its role
  float gam_c[NCB], gb_c[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int kq = cb * 16 + c16;
    const int t = kq < TMAX ? kq : kq - TMAX;
    gam_c[cb] = s_gam[t];
    gb_c[cb] = s_gb[t];
  }
  floatx4 acc1[TPW][NCB];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc1[tt][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    if (TMAX >= 16 && (cb * 16) % TMAX >= T) continue;  // all-padding block
    const float* brow = s_kq + (cb * 16 + c16) * KQ_LD + 4 * kk;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      bf16x8 bhi, blo;
      split_bf16x8(*reinterpret_cast<const floatx4*>(brow + 32 * ks),
                   *reinterpret_cast<const floatx4*>(brow + 32 * ks + 16), bhi, blo);
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt)
        if (wave + tt * kNWave < NTILE)
          acc1[tt][cb] = mfma_bf16x3(shi[tt][ks], slo[tt][ks], bhi, blo, acc1[tt][cb]);
    }
  }
  // RHS_t[i] = b_t (v_t[i] - gamma_t W[i][t]) on the k-row lanes, in place of
  // v (stored [row of S][node]); padding nodes become 0.  Only this wave
  // reads its tiles' RHS back, and a wave's LDS accesses execute in order, so
  // no workgroup barrier separates this from the product below.
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int tile = wave + tt * kNWave;
    if (tile < NTILE) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int kq = cb * 16 + c16;
        if (kq < TMAX) {
          float* col = s_rhs + (tile * 16 + 4 * kk) * RT_LD + kq;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = col[r * RT_LD];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            col[r * RT_LD] = kq < T ? gb_c[cb] * (v[r] - gam_c[cb] * acc1[tt][cb][r]) : 0.f;
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // (10) RHS^T [Ti; M2]^T on MFMA: A = this wave's RHS tile (rows of S x
  //      nodes), B = a 16-row block of [Ti; M2]; block cb's columns are the
  //      same nodes as block cb of the first product, so U (k-row lanes) and
  //      M2 RHS (q-row lanes) land where W and Q S0^T are.
  floatx4 acc2[TPW][NCB];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc2[tt][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
  // A operand of the long-chunk path: this lane's RHS row, split once.
  constexpr int RST = TMAX >= 32 ? TMAX / 32 : 1;
  bf16x8 rhi[TPW][RST], rlo[TPW][RST];
  if constexpr (TMAX >= 32) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int tile = wave + tt * kNWave;
      const float* arow = s_rhs + ((tile < NTILE ? tile : 0) * 16 + c16) * RT_LD + 8 * kk;
#pragma unroll
      for (int st = 0; st < RST; ++st)
        split_bf16x8(*reinterpret_cast<const floatx4*>(arow + 32 * st),
                     *reinterpret_cast<const floatx4*>(arow + 32 * st + 4), rhi[tt][st], rlo[tt][st]);
    }
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    if (TMAX >= 16 && (cb * 16) % TMAX >= T) continue;
    const int brow = cb * 16 + c16;
    const float* bmat = brow < TMAX ? s_Ti + brow * CO_LD : s_G + (brow - TMAX) * CO_LD;
    if constexpr (TMAX >= 32) {
#pragma unroll
      for (int st = 0; st < TMAX / 32; ++st) {
        if (st * 32 >= T) break;
        bf16x8 bhi, blo;
        split_bf16x8(*reinterpret_cast<const floatx4*>(bmat + 32 * st + 8 * kk),
                     *reinterpret_cast<const floatx4*>(bmat + 32 * st + 8 * kk + 4), bhi, blo);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
          if (wave + tt * kNWave < NTILE)
            acc2[tt][cb] = mfma_bf16x3(rhi[tt][st], rlo[tt][st], bhi, blo, acc2[tt][cb]);
      }
    } else {
#pragma unroll
      for (int st = 0; st < TMAX / 4; ++st) {
        if (st * 4 >= T) break;
        const float b_op = bmat[4 * st + kk];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
          const int tile = wave + tt * kNWave;
          if (tile < NTILE) {
            const float a_op = s_rhs[(tile * 16 + c16) * RT_LD + 4 * st + kk];
            acc2[tt][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_op, b_op, acc2[tt][cb], 0, 0, 0);
          }
        }
      }
    }
  }

  // (11) Outputs straight from registers, four consecutive state rows per
  //      lane: u on the k-row lanes, o = gamma Z + M2 RHS on the q-row lanes.
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int tile = wave + tt * kNWave;
    if (tile < NTILE) {
      const int i0 = r0 + tile * 16 + 4 * kk;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int kq = cb * 16 + c16;
        const bool isk = kq < TMAX;
        const int t = isk ? kq : kq - TMAX;
        if (t < T) {
          const size_t oi = ((lb * T + t) * p.Hv + hv) * DV + i0;
          floatx4 val = acc2[tt][cb];
          if (!isk) val += gam_c[cb] * acc1[tt][cb];
          __builtin_nontemporal_store(val, reinterpret_cast<floatx4*>((isk ? p.tu : p.o) + oi));
        }
      }
    }
  }
}

template <int DK, int DV, int TMAX, int ROWS, typename TIn>
hipError_t launch_k(const VerifyArgs& a, int grid, hipStream_t s) {
  if (a.K == 4)
    hipLaunchKernelGGL((k_verify_wy<DK, DV, TMAX, ROWS, 4, TIn>), dim3(grid),
                       dim3(threads_for<TMAX>()), 0, s, a);
  else
    hipLaunchKernelGGL((k_verify_wy<DK, DV, TMAX, ROWS, 0, TIn>), dim3(grid),
                       dim3(threads_for<TMAX>()), 0, s, a);
  return hipGetLastError();
}

template <int DK, int DV, int ROWS, typename TIn>
hipError_t launch_t(const VerifyArgs& a, hipStream_t s);

// fp32 inputs at T > 32 with 128-dim heads use 32-row blocks to stay in LDS.
template <int DK, int DV, int ROWS, typename TIn>
constexpr int rows_for_long() {
  return (sizeof(TIn) == 4 && DV == 128) ? 32 : ROWS;
}

template <int DK, int DV, int ROWS, typename TIn>
hipError_t launch_t(const VerifyArgs& a, hipStream_t s) {
  const int nsub = (a.Hv / a.Hk) * (DV / ROWS);
  const int n_units = a.L * a.B * a.Hk;
  const long long grid = static_cast<long long>((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * nsub;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.T <= 8) return launch_k<DK, DV, 8, ROWS, TIn>(a, static_cast<int>(grid), s);
  if (a.T <= 16) return launch_k<DK, DV, 16, ROWS, TIn>(a, static_cast<int>(grid), s);
  if (a.T <= 32) return launch_k<DK, DV, 32, ROWS, TIn>(a, static_cast<int>(grid), s);
  constexpr int RL = rows_for_long<DK, DV, ROWS, TIn>();
  if constexpr (RL != ROWS) {
    const int nsub2 = (a.Hv / a.Hk) * (DV / RL);
    const long long grid2 = static_cast<long long>((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * nsub2;
    if (grid2 > 0x7fffffffLL) return hipErrorInvalidValue;
    return launch_k<DK, DV, 64, RL, TIn>(a, static_cast<int>(grid2), s);
  } else {
    return launch_k<DK, DV, 64, ROWS, TIn>(a, static_cast<int>(grid), s);
  }
}

template <typename TIn>
hipError_t launch_d(const VerifyArgs& a, int dk, int dv, hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 32: return launch_t<32, 32, 32, TIn>(a, s);
    case 64: return launch_t<64, 64, 64, TIn>(a, s);
    case 128: return launch_t<128, 128, 128, TIn>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_verify_wy(const VerifyArgs& a, int dk, int dv, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_d<uint16_t>(a, dk, dv, s) : launch_d<float>(a, dk, dv, s);
}

}  // namespace gdn
