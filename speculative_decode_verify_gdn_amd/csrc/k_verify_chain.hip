// k_verify_chain.hip -- verify of a short drafted chain (T <= 16 tokens)
// through one GDN layer, for gfx950, with one wave specialised for the
// per-head prologue and the others for the state.
//
// Same algebra as the chunked form in k_verify_wy.hip (GDN page s2.1, the
// delta rule unrolled over the chunk; replay form in s4), for a chain:
//   gamma_t = a_0 ... a_t,  Gamma[t,i] = a_{i+1} ... a_t
//   A[t,i]  = b_t Gamma[t,i] k_t.k_i (i < t),  Oc[t,i] = Gamma[t,i] q_t.k_i (i <= t)
//   Ti = (I + A)^-1,  M2 = Oc Ti,  RHS_t = b_t (v_t - gamma_t S0 k_t)
//   U = Ti RHS,  O = diag(gamma) Q S0^T + M2 RHS.
// q and k are L2-normalised after the conv.  Here the normalisation is a
// scale: the Gram of the raw (post-conv) rows gives the norms on its
// diagonal, and the state products use the raw rows with the per-node
// scales r_t = 1/sqrt(|x_t|^2 + eps) applied to their fp32 results.
//
// Why wave 0 works alone first.  A wave that has queued 16 KiB of state
// loads cannot issue further instructions until the memory pipeline has
// accepted them, which under full load takes most of the time the state
// takes to arrive.  So:
//   wave 0 issues only the small loads (raw conv rows, weights, gates), then
//     -- with no workgroup barrier -- does conv + SiLU, the Gram of [K;Q] on
//     bf16x3 MFMA, the norms and the T x T algebra, and leaves the pre-split
//     K/Q operands, V, [Ti;M2] and per-node scales in LDS;
//   waves 1.. wait only until wave 0 has issued its loads, then queue their
//     whole share of S0 at once;
//   after one barrier every wave runs S0 [K;Q]^T (bf16x3 MFMA), the RHS,
//     RHS [Ti;M2]^T (fp32 MFMA) and stores u and o from registers; wave 0
//     queues its own share of S0 only then, so it arrives last.
// Workgroups of four waves pack four to a CU: a fifth, state-less prologue
// wave would put two waves of one workgroup on a SIMD and leave a quarter of
// the workgroups waiting for a free slot.  (Measured alternatives -- a
// prologue-only wave with the state on three waves, raised issue priority
// for the prologue, delaying the state loads -- were no faster.)
// S0 and the conv window are never written (they stay the snapshot), except
// by the forms below.
//
// Forms (template flags): RP folds the previous round's accepted prefix into
// S first (the rank-n tape replay on fp32 MFMA, written back in place); VG
// takes the decay gate per key channel (the walk that forms the A and Oc
// coefficients from forward gate products, and per-channel weights on the k
// operand of the replay); PF walks a whole prefill through the workgroup in
// chunks of TMAX tokens with the state held in registers.
//
// Work item: one workgroup per (layer, seq, v-head), all Dv rows of S.

#include "gdn_common.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {


template <int DV>
constexpr int chain_waves() {
  return DV / 16 < 4 ? DV / 16 : 4;
}
template <int DV>
constexpr int chain_threads() {
  return 64 * chain_waves<DV>();
}

// Split two fp32 values into packed bf16 high parts and residuals, one
// conversion per value: fewer values live than the paired split, which the
// prefill loop needs at its register limit.
__device__ __forceinline__ void split_pair_each(float y0, float y1, uint32_t& hi, uint32_t& lo) {
  const __bf16 h0 = static_cast<__bf16>(y0);
  const __bf16 h1 = static_cast<__bf16>(y1);
  bf16x2 h = {h0, h1};
  bf16x2 l = {static_cast<__bf16>(y0 - static_cast<float>(h0)),
              static_cast<__bf16>(y1 - static_cast<float>(h1))};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

// Sum over aligned groups of 16 lanes (DPP; every lane gets its group's sum).
__device__ __forceinline__ float sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ float silu_f(float y) {
  return y * __builtin_amdgcn_rcpf(1.f + __expf(-y));
}

// Two adjacent input elements widened to fp32.
template <typename TIn>
struct Pair;
template <>
struct Pair<uint16_t> {
  typedef uint32_t raw;
  static __device__ __forceinline__ raw load(const uint16_t* p) {
    return *reinterpret_cast<const uint32_t*>(p);
  }
  static __device__ __forceinline__ float lo(raw r) { return __uint_as_float(r << 16); }
  static __device__ __forceinline__ float hi(raw r) { return __uint_as_float(r & 0xffff0000u); }
};
template <>
struct Pair<float> {
  typedef floatx2 raw;
  static __device__ __forceinline__ raw load(const float* p) {
    return *reinterpret_cast<const floatx2*>(p);
  }
  static __device__ __forceinline__ float lo(raw r) { return r[0]; }
  static __device__ __forceinline__ float hi(raw r) { return r[1]; }
};

// Sequence at position q of the order that lists first the sequences with a
// previous prefix to replay (1 <= prev_n_keep[b] <= pT), then the others,
// each group in index order.  Every lane of the wave takes part; the result
// is wave-uniform.
__device__ __forceinline__ int writers_first_seq(const int32_t* pnk, int B, int pT, int q) {
  const int lane = threadIdx.x & (kWave - 1);
  int W = 0;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int b = c0 + lane;
    const int v = b < B ? pnk[b] : 0;
    W += __popcll(__ballot(b < B && v >= 1 && v <= pT));
  }
  const bool want = q < W;
  int target = want ? q : q - W;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int b = c0 + lane;
    const int v = b < B ? pnk[b] : 0;
    const bool wr = v >= 1 && v <= pT;
    unsigned long long m = __ballot(b < B && wr == want);
    const int cnt = __popcll(m);
    if (target < cnt) {
      for (int k = 0; k < target; ++k) m &= m - 1ull;
      return c0 + __builtin_ctzll(m);
    }
    target -= cnt;
  }
  return q;  // not reached for q < B
}

template <int DK, int DV, int TMAX, int KM, typename TIn>
struct ChainLayout {
  static constexpr int NW = chain_waves<DV>();
  static constexpr int NT = chain_threads<DV>();
  static constexpr int NTILE = DV / 16;
  static constexpr int TPW = NTILE / NW;  // 16-row tiles per wave
  static_assert(NTILE % NW == 0, "tiles per wave");
  static constexpr int NKQ = 2 * TMAX;          // k rows [0,TMAX), q rows [TMAX,2TMAX)
  static constexpr int KQS = 4 * DK + 16;       // bytes per pre-split row (+16: conflict-free b128)
  static constexpr int RT_LD = TMAX + 1;        // V / RHS, [row of S][node]
  static constexpr int GLD = NKQ + 1;           // Gram
  static constexpr int ALD = NKQ + 1;           // A, Oc (in place of the Gram rows)
  static constexpr int BLD = TMAX + 1;          // [Ti; M2]
  static constexpr int NPAIR = (2 * DK + DV) / 2;
  static constexpr int PPL = (NPAIR + 63) / 64;  // channel pairs per prologue lane
  static constexpr int XR = TMAX + KM - 1;       // raw rows: old window + tokens
  static constexpr int RAW_WORDS = PPL * XR * (int)sizeof(TIn) / 2;
  static constexpr bool LOAD_ALL = RAW_WORDS + PPL * 2 * KM <= 96;
  static_assert(DK % 32 == 0 && DV % 16 == 0 && (TMAX == 8 || TMAX == 16), "tiling");
  static constexpr int KF = TMAX * DK > NKQ * BLD ? TMAX * DK : NKQ * BLD;  // raw k rows, then [Ti; M2]
  static_assert(ALD == GLD, "A and Oc overwrite the Gram rows in place");
};

// Occupancy targets.  PF (prefill loop) holds the state across the
// prologue: with the per-head gate it runs at 3 waves per SIMD (166 VGPRs,
// no spill at conv width 4), measured faster than 2 and far faster than 4
// (heavy spill); with the per-key gate at 2 (no spill), faster than 3
// (spill).  The per-key replay (VG and RP) runs at 3, spill-free.
template <int DK, int DV, int TMAX, int KC, typename TIn, bool RP, bool VG = false, bool PF = false>
__global__ __launch_bounds__(chain_threads<DV>())
__attribute__((amdgpu_waves_per_eu(PF && VG ? 2 : (PF || (VG && RP) ? 3 : 4)))) void k_verify_chain(VerifyArgs p0) {
  static_assert(!PF || RP, "the prefill loop runs the replay form");
  static_assert(!VG || (DK == 128 && DV == 128 && sizeof(TIn) == 2),
                "the per-key-channel gate runs 128-dim heads, bf16 inputs");
  constexpr int KM = KC > 0 ? KC : 8;
  using LY = ChainLayout<DK, DV, TMAX, KM, TIn>;
  using PR = Pair<TIn>;
  constexpr int NW = LY::NW, TPW = LY::TPW, NKQ = LY::NKQ, KQS = LY::KQS;
  constexpr int RT_LD = LY::RT_LD, GLD = LY::GLD, ALD = LY::ALD, BLD = LY::BLD;
  constexpr int NPAIR = LY::NPAIR, PPL = LY::PPL, XR = LY::XR;
  constexpr int KSTEPS = DK / 32;
  constexpr int NCB = NKQ / 16;  // 16-column blocks of [K;Q]

  __shared__ __align__(16) unsigned char s_kq[NKQ * KQS];  // pre-split raw k, q rows
  __shared__ __align__(16) float s_kf[LY::KF];             // raw k rows (fp32) for the tape, then [Ti; M2]
  __shared__ __align__(16) float s_rhs[DV * RT_LD];        // v, then RHS
  __shared__ float s_G[NKQ * GLD];                         // Gram, then A (k rows) and Oc (q rows) in place
  float* const s_A = s_G;
  float* const s_Oc = s_G + TMAX * GLD;
  float* const s_B = s_kf;                                 // rows: Ti, then M2
  __shared__ float s_rn[NKQ], s_ga[TMAX], s_gb[TMAX];
  __shared__ float s_ck[TMAX], s_cq[TMAX], s_cb[TMAX];
  // per-key-channel gates [token][channel], bf16 as given
  __shared__ __align__(16) uint16_t s_av[VG ? TMAX * DK : 8];
  // previous round's accepted prefix: w_i = prod_{i<j<pn} g_j (zero for
  // i >= pn) and gamma = prod_{j<pn} g_j
  constexpr int PM = 16;
  __shared__ float s_pw[RP ? PM : 1];
  __shared__ float s_pgam;
  // per-key-channel replay: w_{i,c} = prod_{i<j<pn} g_{j,c} (zero for i >= pn)
  // as [i][c], and gamma_c = prod_{j<pn} g_{j,c}
  constexpr bool VR = VG && RP;
  __shared__ float s_pwk[VR ? PM * DK : 1];
  __shared__ __align__(16) float s_pgk[VR ? DK : 4];
  // prefill loop, bf16 and conv width 4: the next chunk's raw conv rows,
  // [row][channel pair], fetched by the last wave while wave 0 solves
  constexpr bool PFX = PF && sizeof(TIn) == 2 && KC == 4;
  __shared__ typename PR::raw s_raw[PFX ? XR * NPAIR : 1];

  const int G = p0.Hv / p0.Hk;
  const int n_units = p0.L * p0.B * p0.Hk;
  const UnitSub us = xcd_unit_sub(blockIdx.x, G);
  if (us.unit >= n_units) return;
  const int hk = us.unit % p0.Hk;
  size_t lb = us.unit / p0.Hk;  // l * B + b
  const int l = static_cast<int>(lb / p0.B);
  if constexpr (RP && !PF) {
    // The sequences that replay (and write their state back) go first, so
    // that one pass of workgroups over the CUs (workgroup i on CU i mod the
    // CU count) spreads them evenly instead of letting a CU draw several.
    // Larger batches run many passes, which even out by themselves.  The
    // per-key form keeps index order: at three waves per SIMD its rounds run
    // several passes at every batch size, and the reordering measured slower
    // there (256 sequences: 356 against 327 us per layer).
    if (!VG && p0.prev_n_keep && p0.B <= 256) {
      const int q = static_cast<int>(lb % p0.B);
      lb = static_cast<size_t>(l) * p0.B + writers_first_seq(p0.prev_n_keep, p0.B, p0.pT, q);
    }
  }
  const int g = us.sub;
  const int hv = hk * G + g;
  // This wave's tiles of S0 (tile wave + tt * NW): lane (c16, kk) holds row
  // c16 of a tile, columns 16m + 4kk .. +3, as MFMA A operands.  The prefill
  // loop carries them across chunks.
  typedef floatx4 SregT[TPW][DK / 16];
  SregT sreg_pf;

  // Prefill (PF): the workgroup runs all T tokens as chunks of TMAX with the
  // state held in registers.  Chunk c is verified from the state after
  // chunks 0 .. c-1 and writes its tape to slot c % 2 of the workspace (the
  // tu/tk/tg and ptu/ptk/ptg pointers); the next chunk first folds it into
  // the state with the replay update, every token kept.  S is read before the
  // first chunk and written after the last; the conv window of chunk c > 0 is
  // the previous chunk's last raw rows, read in place from x.
  // Without PF the body runs once: the exit test sits at its end, so that the
  // single pass compiles as straight-line code.
  const int nch = PF ? (p0.T + TMAX - 1) / TMAX : 1;
  for (int ch = 0;; ++ch) {
  VerifyArgs pl = p0;  // this chunk's view (prefill)
  if constexpr (PF) {
    // Opaque per-chunk copies of the loop-invariant operands, so that the
    // compiler rematerialises what derives from them inside each chunk
    // instead of keeping it live in registers across the whole loop.
    const float* cw = p0.conv_w;
    int hkn = p0.Hk, hvn = p0.Hv, cn = p0.C;
    asm volatile("" : "+s"(cw), "+s"(hkn), "+s"(hvn), "+s"(cn));
    pl.conv_w = cw;
    pl.Hk = hkn;
    pl.Hv = hvn;
    pl.C = cn;
    const int c0 = ch * TMAX;
    const size_t C = p0.C;
    pl.T = p0.T - c0 < TMAX ? p0.T - c0 : TMAX;
    pl.x = static_cast<const TIn*>(p0.x) + c0 * C;
    pl.a = static_cast<const TIn*>(p0.a) + static_cast<size_t>(c0) * p0.Hv * (VG ? DK : 1);
    pl.b = static_cast<const TIn*>(p0.b) + static_cast<size_t>(c0) * p0.Hv;
    pl.o = p0.o + static_cast<size_t>(c0) * p0.Hv * DV;
    if (ch > 0) {
      pl.conv_state = static_cast<const TIn*>(p0.x) + (c0 - (KC > 0 ? KC : p0.K) + 1) * C;
      pl.cs_ld = p0.x_ld;
    }
    const bool odd = ch & 1;
    pl.tu = odd ? const_cast<float*>(p0.ptu) : p0.tu;
    pl.tk = odd ? const_cast<float*>(p0.ptk) : p0.tk;
    pl.tg = odd ? const_cast<float*>(p0.ptg) : p0.tg;
    pl.ptu = odd ? p0.tu : p0.ptu;
    pl.ptk = odd ? p0.tk : p0.ptk;
    pl.ptg = odd ? p0.tg : p0.ptg;
    pl.prev_n_keep = nullptr;
    pl.prev_n_all = ch > 0 ? TMAX : 0;
    pl.pT = TMAX;
  }
  const VerifyArgs& p = PF ? pl : p0;
  SregT sreg_own;
  SregT& sreg = PF ? sreg_pf : sreg_own;
  int tid_l = threadIdx.x;
  if constexpr (PF) asm volatile("" : "+v"(tid_l));  // per-chunk lane addressing
  const int tid = tid_l;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int kk = lane >> 4;
  const int T = p.T;
  const int K = KC > 0 ? KC : p.K;
  // accepted length of the previous round (replay variant)
  int pn = 0;
  if constexpr (RP) {
    const int bb = static_cast<int>(lb % p.B);
    const int v = p.prev_n_keep ? p.prev_n_keep[bb] : p.prev_n_all;
    pn = (v >= 0 && v <= p.pT && v <= PM) ? v : 0;
    if (pn != v && tid == 0 && p.dev_err && l == 0 && hk == 0 && g == 0)
      atomicOr(p.dev_err, GDN_DEV_ERR_N_KEEP);
  }

  const float* S_head = p.S + (lb * p.Hv + hv) * static_cast<size_t>(DV * DK);
  float* const S_live = RP ? p.S_out + (lb * p.Hv + hv) * static_cast<size_t>(DV * DK) : nullptr;
  // Replay operands, straight from the previous tape into registers: lane
  // (c16, kk) takes k_i[16m + c16] (A) and u_i[16 tile + c16] (B) for
  // i = 4 st + kk.  Steps with 4 st >= pn are skipped (pn is uniform).
  float kt[RP ? PM / 4 : 1][RP ? DK / 16 : 1];
  float ut[RP ? TPW : 1][RP ? PM / 4 : 1];
  auto load_tape = [&]() {
    if constexpr (RP) {
      const size_t base = lb * p.pT;
#pragma unroll
      for (int st = 0; st < PM / 4; ++st) {
        if (4 * st < pn) {
          const int i = 4 * st + kk;
          const size_t ii = base + (i < pn ? i : 0);
          const float* kr = p.ptk + (PF ? ii * p.Hv + hv : ii * p.Hk + hk) * DK + c16;
#pragma unroll
          for (int m = 0; m < DK / 16; ++m) kt[st][m] = kr[16 * m];
          const float* ur = p.ptu + (ii * p.Hv + hv) * DV + c16;
#pragma unroll
          for (int tt = 0; tt < TPW; ++tt) ut[tt][st] = ur[(wave + tt * NW) * 16];
        }
      }
    }
  };
  auto load_state = [&]() {
    if (PF && ch > 0) return;  // the state is in registers
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const float* rp = S_head + static_cast<size_t>((wave + tt * NW) * 16 + c16) * DK + 4 * kk;
#pragma unroll
      for (int m = 0; m < DK / 16; ++m) sreg[tt][m] = *reinterpret_cast<const floatx4*>(rp + 16 * m);
    }
  };

  // Conv helpers (prologue).  Wave 0 runs every channel pair in the verify
  // forms; the prefill loop shares the pairs out over the waves, since from
  // its second chunk on the state waves have no loads to queue.
  const TIn* x = static_cast<const TIn*>(p.x);
  const TIn* cs = static_cast<const TIn*>(p.conv_state);
  const float* cw = p.conv_w + static_cast<size_t>(l) * p.C * K;
  const TIn* xcol = x + lb * p.x_ld;
  const TIn* ccol = cs + lb * (PF ? p.cs_ld : static_cast<size_t>(K - 1) * p.C);
  const int nrows = K - 1 + T;
  // local channel c in [q | k | v-rows] -> qkv channel
  auto chan = [&](int c) {
    return c < DK ? hk * DK + c
                  : (c < 2 * DK ? p.Hk * DK + hk * DK + (c - DK)
                                : 2 * p.Hk * DK + hv * DV + (c - 2 * DK));
  };
  const bool raw_lds = PFX && ch > 0;  // rows fetched ahead into s_raw
  auto load_pair = [&](int j, typename PR::raw* xr, float* w0, float* w1) {
    const int pr = lane + 64 * j;
    const int c0 = 2 * (pr < NPAIR ? pr : NPAIR - 1);
    const int ch = chan(c0);
#pragma unroll
    for (int r = 0; r < XR; ++r) {
      const int rr = r < nrows ? r : nrows - 1;
      const TIn* base = rr < K - 1 ? ccol + static_cast<size_t>(rr) * p.C
                                   : xcol + static_cast<size_t>(rr - (K - 1)) * p.C;
      xr[r] = raw_lds ? s_raw[r * NPAIR + c0 / 2] : PR::load(base + ch);
    }
    if (KC == 4) {
      const floatx4 a0 = *reinterpret_cast<const floatx4*>(cw + static_cast<size_t>(ch) * 4);
      const floatx4 a1 = *reinterpret_cast<const floatx4*>(cw + static_cast<size_t>(ch) * 4 + 4);
#pragma unroll
      for (int jj = 0; jj < KM; ++jj) {
        w0[jj] = a0[jj % 4];
        w1[jj] = a1[jj % 4];
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < KM; ++jj) {
        const int q = jj < K ? jj : 0;
        const float v0 = cw[static_cast<size_t>(ch) * K + q];
        const float v1 = cw[static_cast<size_t>(ch + 1) * K + q];
        w0[jj] = jj < K ? v0 : 0.f;
        w1[jj] = jj < K ? v1 : 0.f;
      }
    }
  };
  // conv + SiLU of one channel pair over the chunk; results to LDS.
  auto conv_pair = [&](int j, const typename PR::raw* xr, const float* w0, const float* w1) {
    const int pr = lane + 64 * j;
    if (pr >= NPAIR) return;
    const int c0 = 2 * pr;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      float y0 = 0.f, y1 = 0.f;
#pragma unroll
      for (int jj = 0; jj < KM; ++jj) {
        if (t + jj < XR) {
          y0 = fmaf(w0[jj], PR::lo(xr[t + jj]), y0);
          y1 = fmaf(w1[jj], PR::hi(xr[t + jj]), y1);
        }
      }
      if (p.silu) {
        y0 = silu_f(y0);
        y1 = silu_f(y1);
      }
      if (t >= T) y0 = y1 = 0.f;
      if (c0 < 2 * DK) {
        const int isq = c0 < DK;
        const int c = isq ? c0 : c0 - DK;
        const int n = isq ? TMAX + t : t;
        // element c -> 32-column step s, half h, lane group kg, slot e
        const int s = c / 32, h = (c % 32) / 16, kg = (c % 16) / 4, e = c % 4;
        unsigned char* row = s_kq + n * KQS + s * 128 + kg * 32 + (h * 4 + e) * 2;
        uint32_t hi, lo;
        split_pair_each(y0, y1, hi, lo);
        *reinterpret_cast<uint32_t*>(row) = hi;
        *reinterpret_cast<uint32_t*>(row + 16) = lo;
        if (!isq) *reinterpret_cast<floatx2*>(s_kf + t * DK + c) = floatx2{y0, y1};
      } else {
        const int i = c0 - 2 * DK;
        s_rhs[i * RT_LD + t] = y0;
        s_rhs[(i + 1) * RT_LD + t] = y1;
      }
    }
  };

  // Per-key gate: the walk that forms row t of A and Oc (see the per-key
  // block of the prologue) for one token, on one 16-lane group (channels
  // 8 li .. 8 li + 7 per lane).  A token's walk writes only its own rows.
    const int gq = lane >> 4, li = lane & 15;
    auto read_pre = [&](int n, float* y) {  // channels 8 li .. +7 of pre-split row n
      const unsigned char* row = s_kq + n * KQS + (li / 4) * 128 + ((li % 4) / 2) * 8;
      const int kg = 2 * (li % 2);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint2 hi = *reinterpret_cast<const uint2*>(row + (kg + hf) * 32);
        const uint2 lo = *reinterpret_cast<const uint2*>(row + (kg + hf) * 32 + 16);
        y[4 * hf] = __uint_as_float(hi.x << 16) + __uint_as_float(lo.x << 16);
        y[4 * hf + 1] = __uint_as_float(hi.x & 0xffff0000u) + __uint_as_float(lo.x & 0xffff0000u);
        y[4 * hf + 2] = __uint_as_float(hi.y << 16) + __uint_as_float(lo.y << 16);
        y[4 * hf + 3] = __uint_as_float(hi.y & 0xffff0000u) + __uint_as_float(lo.y & 0xffff0000u);
      }
    };
    auto write_pre = [&](int n, const float* y) {
      unsigned char* row = s_kq + n * KQS + (li / 4) * 128 + ((li % 4) / 2) * 8;
      const int kg = 2 * (li % 2);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint32_t h0, l0, h1, l1;
        split_pair_each(y[4 * hf], y[4 * hf + 1], h0, l0);
        split_pair_each(y[4 * hf + 2], y[4 * hf + 3], h1, l1);
        *reinterpret_cast<uint2*>(row + (kg + hf) * 32) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(row + (kg + hf) * 32 + 16) = make_uint2(l0, l1);
      }
    };
    auto gates8 = [&](int t, float* a) {
      const u32x4 r = *reinterpret_cast<const u32x4*>(s_av + t * DK + 8 * li);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        a[2 * w] = __uint_as_float(r[w] << 16);
        a[2 * w + 1] = __uint_as_float(r[w] & 0xffff0000u);
      }
    };
    auto kn8 = [&](int t, float* k) {  // normalised k of token t
      const floatx4 k0 = *reinterpret_cast<const floatx4*>(s_kf + t * DK + 8 * li);
      const floatx4 k1 = *reinterpret_cast<const floatx4*>(s_kf + t * DK + 8 * li + 4);
      const float r = s_rn[t];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k[e] = k0[e] * r;
        k[4 + e] = k1[e] * r;
      }
    };
  // Rows i in [lo, hi) of token t (hi <= t): the rows above hi only
  // advance the gate product.  `last` also finishes the token: its diagonal
  // Oc entry and the gamma-scaled operand rows.
  auto walk_part = [&](int t, int lo, int hi, bool last) {
    if (t < T) {
      float kv[8], qv[8], w[8];
      kn8(t, kv);
      read_pre(TMAX + t, qv);
      const float rq = s_rn[TMAX + t];
      float kq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qv[e] *= rq;
        kq = fmaf(kv[e], qv[e], kq);
      }
      gates8(t, w);
      const float bt = s_gb[t];
      for (int i = t - 1; i >= hi; --i) {
        float ai[8];
        gates8(i, ai);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] *= ai[e];
      }
      for (int i = hi - 1; i >= lo; --i) {
        float ki[8], ai[8];
        kn8(i, ki);
        gates8(i, ai);
        float cc = 0.f, dd = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kw = ki[e] * w[e];
          cc = fmaf(kw, kv[e], cc);
          dd = fmaf(kw, qv[e], dd);
          w[e] *= ai[e];
        }
        cc = sum16(cc);
        dd = sum16(dd);
        if (li == 0) {
          s_A[t * ALD + i] = bt * cc;
          s_Oc[t * ALD + i] = dd;
        }
      }
      if (last) {
        kq = sum16(kq);
        if (li == 0) s_Oc[t * ALD + t] = kq;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kv[e] *= w[e];
          qv[e] *= w[e];
        }
        write_pre(t, kv);
        write_pre(TMAX + t, qv);
      }
    }
  };
  // The prefill loop's share for 16-lane group g = 4 wave + gq: the upper
  // half of token g's walk and the lower half of token 15 - g's (at most 8
  // full steps a group; the walk of token t has t).
  auto walk_share = [&](int g) {
    walk_part(g, (g + 1) / 2, g, false);
    walk_part(15 - g, 0, (16 - g) / 2, true);
  };
  if (wave == 0) {
    // ---------------------------------------------------------- prologue --
    // Gates (clamped, unconditional loads).
    const int tq = lane < T ? lane : 0;
    const size_t gi = lb * p.ab_ld + static_cast<size_t>(tq) * p.Hv + hv;
    // (the per-key-channel gate enters through the operands instead)
    const float ga_ld = VG ? 1.f : ld_in(static_cast<const TIn*>(p.a), gi);
    const float gb_ld = ld_in(static_cast<const TIn*>(p.b), gi);
    // per-key-channel gates: lane takes 16-byte chunks lane + 64 j, chunk q
    // holding channels 8 (q % 16) .. +7 of token q / 16
    constexpr int NAV = VG ? (TMAX * DK / 8 + 63) / 64 : 1;
    u32x4 avr[NAV];
    if constexpr (VG) {
#pragma unroll
      for (int j = 0; j < NAV; ++j) {
        const int q = lane + 64 * j;
        const int t = q / (DK / 8);
        const uint16_t* ap = static_cast<const uint16_t*>(p.a) +
                             (lb * p.ab_ld + static_cast<size_t>(t < T ? t : 0) * p.Hv + hv) * DK +
                             8 * (q % (DK / 8));
        avr[j] = *reinterpret_cast<const u32x4*>(ap);
      }
    }
    const float pg_ld = RP && !VG && lane < pn ? p.ptg[(lb * p.pT + lane) * p.Hv + hv] : 1.f;


    if constexpr (PF) {
      // this wave's share of the channel pairs, then (B0') every wave's
      // conv results are in LDS
      for (int j = 0; j < PPL; j += NW) {
        typename PR::raw xr[XR];
        float w0[KM], w1[KM];
        load_pair(j, xr, w0, w1);
        conv_pair(j, xr, w0, w1);
      }
      __syncthreads();  // (B0')
    } else if constexpr (LY::LOAD_ALL) {
      typename PR::raw xr[PPL][XR];
      float w0[PPL][KM], w1[PPL][KM];
#pragma unroll
      for (int j = 0; j < PPL; ++j) load_pair(j, xr[j], w0[j], w1[j]);
      __syncthreads();  // (B0) every small load is queued ahead of the state
#pragma unroll
      for (int j = 0; j < PPL; ++j) conv_pair(j, xr[j], w0[j], w1[j]);
    } else {
      __syncthreads();  // (B0)
#pragma unroll 1
      for (int j = 0; j < PPL; ++j) {
        typename PR::raw xr[XR];
        float w0[KM], w1[KM];
        load_pair(j, xr, w0, w1);
        conv_pair(j, xr, w0, w1);
      }
    }
    if constexpr (RP && !VG) {
      float w = 1.f, gm = 1.f;
#pragma unroll
      for (int j = 0; j < PM; ++j) {
        const float gj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pg_ld), j));
        gm *= gj;
        if (j > lane) w *= gj;
      }
      if (lane < PM) s_pw[lane] = lane < pn ? w : 0.f;
      if (lane == 0) s_pgam = gm;
    }
    if (lane < TMAX) {
      s_ga[lane] = lane < T ? ga_ld : 1.f;
      s_gb[lane] = lane < T ? gb_ld : 0.f;
      if (lane < T && !VG) p.tg[(lb * T + lane) * p.Hv + hv] = ga_ld;
    }
    if constexpr (VG) {
#pragma unroll
      for (int j = 0; j < NAV; ++j) {
        const int q = lane + 64 * j;
        const int t = q / (DK / 8), c0 = 8 * (q % (DK / 8));
        if (t < TMAX) *reinterpret_cast<u32x4*>(s_av + t * DK + c0) = avr[j];
        if (t < T) {
          floatx4 v0, v1;
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            v0[2 * w] = __uint_as_float(avr[j][w] << 16);
            v0[2 * w + 1] = __uint_as_float(avr[j][w] & 0xffff0000u);
            v1[2 * w] = __uint_as_float(avr[j][2 + w] << 16);
            v1[2 * w + 1] = __uint_as_float(avr[j][2 + w] & 0xffff0000u);
          }
          floatx4* tgp = reinterpret_cast<floatx4*>(p.tg + ((lb * T + t) * p.Hv + hv) * DK + c0);
          tgp[0] = v0;
          tgp[1] = v1;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // Gram G' = [K;Q][K;Q]^T of the raw rows on bf16x3 MFMA (lower tiles).
#pragma unroll
    for (int rb = 0; rb < NCB; ++rb) {
#pragma unroll
      for (int cb = 0; cb <= rb; ++cb) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        const unsigned char* ar = s_kq + (rb * 16 + c16) * KQS + kk * 32;
        const unsigned char* br = s_kq + (cb * 16 + c16) * KQS + kk * 32;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(ar + s * 128);
          const bf16x8 alo = *reinterpret_cast<const bf16x8*>(ar + s * 128 + 16);
          const bf16x8 bhi = *reinterpret_cast<const bf16x8*>(br + s * 128);
          const bf16x8 blo = *reinterpret_cast<const bf16x8*>(br + s * 128 + 16);
          acc = mfma_bf16x3(ahi, alo, bhi, blo, acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) s_G[(rb * 16 + 4 * kk + r) * GLD + cb * 16 + c16] = acc[r];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < NKQ) {
      const float d = s_G[lane * GLD + lane];
      s_rn[lane] = (lane % TMAX) < T ? 1.f / sqrtf(d + p.eps) : 0.f;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // Tape k: the normalised k rows, once per k-head (before [Ti; M2] takes
    // their space).  The prefill loop reads its own chunk tapes back while the
    // k-head's other workgroups run at their own pace, so there every
    // workgroup keeps its own copy, per v-head.
    if (PF || g == 0) {
      constexpr int C4 = DK / 4;
      for (int e = lane; e < T * C4; e += 64) {
        const int t = e / C4, c4 = e % C4;
        const floatx4 v = *reinterpret_cast<const floatx4*>(s_kf + t * DK + 4 * c4) * s_rn[t];
        const size_t row = PF ? (lb * T + t) * p.Hv + hv : (lb * T + t) * p.Hk + hk;
        __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(p.tk + row * DK) + c4);
      }
    }

    // prefill loop, per-head gate: this lane's A and Oc entries (see below)
    constexpr int NQ = TMAX * TMAX / 64;
    float cav[VG || !PF ? 1 : NQ], cov[VG || !PF ? 1 : NQ];
    if constexpr (VG) {
      // Per-key-channel gate: token t's state before it, applied to a_t * k_t,
      // is S0 (gamma_t * k_t) + sum_{i<t} u_i c_{t,i} with c_{t,i} =
      // sum_c k_i[c] w_{t,i}[c] k_t[c], w_{t,i} the product of a_j over
      // i < j <= t and gamma_t over j <= t; o_t adds d_{t,i} (q_t in place of
      // k_t) and u_t (k_t . q_t).  So A[t,i] = b_t c_{t,i} and Oc[t,i] =
      // d_{t,i}, found by walking back from t (only forward gate products),
      // and the operand rows become gamma_t * k_t and gamma_t * q_t
      // (normalised), leaving the per-token scales at b_t and 1.
      for (int e = lane; e < 2 * TMAX * ALD; e += 64) s_G[e] = 0.f;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if constexpr (PF) {
        // the prefill loop shares the walks out over the waves (the other
        // waves have no state to load), halves of two tokens per group
        static_assert(!PF || (TMAX == 16 && NW == 4), "four tokens per wave");
        __syncthreads();  // (B_w0) norms, gates and zeroed A/Oc in LDS
        walk_share(gq);
        __syncthreads();  // (B_w1) every token's walk is done
      } else {
        // 16-lane group gq takes tokens paired for equal walks
#pragma unroll
        for (int j = 0; j < TMAX / 4; ++j)
        {
          const int t = (j % 2 == 0) ? 8 * (j / 2) + gq : 8 * (j / 2) + 7 - gq;
          walk_part(t, 0, t, true);
        }
      }
      if (lane < TMAX) {
        const bool live = lane < T;
        s_ck[lane] = live ? s_gb[lane] : 0.f;
        s_cq[lane] = live ? 1.f : 0.f;
        s_cb[lane] = live ? s_gb[lane] : 0.f;
      }
    } else {
      // T x T coefficients, (t, i) pairs over the lanes, each written in
      // place of the Gram entries it reads (prefill loop: entry e = t TMAX + i
      // of A and Oc stays in register e / 64 of lane e % 64).
      float ga[TMAX];
#pragma unroll
      for (int s = 0; s < TMAX; ++s) ga[s] = s_ga[s];
#pragma unroll
      for (int q = 0; q < TMAX * TMAX / 64; ++q) {
        const int e = lane + 64 * q;
        const int t = e / TMAX, i = e % TMAX;
        float gm = 1.f;  // Gamma[t,i] = a_{i+1} ... a_t
#pragma unroll
        for (int s = 0; s < TMAX; ++s) gm *= (s > i && s <= t) ? ga[s] : 1.f;
        const float rki = s_rn[i];
        const float av = s_gb[t] * gm * s_G[t * GLD + i] * s_rn[t] * rki;
        const float ov = gm * s_G[(TMAX + t) * GLD + i] * s_rn[TMAX + t] * rki;
        if constexpr (PF) {
          cav[q] = (t < T && i < t) ? av : 0.f;
          cov[q] = (t < T && i <= t) ? ov : 0.f;
        } else {
          s_A[t * ALD + i] = (t < T && i < t) ? av : 0.f;
          s_Oc[t * ALD + i] = (t < T && i <= t) ? ov : 0.f;
        }
      }
      if (lane < TMAX) {
        float gm = 1.f;  // gamma_t = a_0 ... a_t
#pragma unroll
        for (int s = 0; s < TMAX; ++s) gm *= s <= lane ? ga[s] : 1.f;
        const bool live = lane < T;
        s_ck[lane] = live ? s_gb[lane] * gm * s_rn[lane] : 0.f;
        s_cq[lane] = live ? gm * s_rn[TMAX + lane] : 0.f;
        s_cb[lane] = live ? s_gb[lane] : 0.f;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // Ti = (I + A)^-1 and M2 = Oc Ti, column j per lane, in registers.
    if constexpr (VG || !PF) {
      if (lane < TMAX) {
        const int j = lane;
        float xc[TMAX];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
          float v = (t == j) ? 1.f : 0.f;
#pragma unroll
          for (int a = 0; a < t; ++a) v = fmaf(-s_A[t * ALD + a], xc[a], v);
          xc[t] = (t < T && j < T) ? v : 0.f;
        }
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
          float m = 0.f;
#pragma unroll
          for (int a = 0; a <= t; ++a) m = fmaf(s_Oc[t * ALD + a], xc[a], m);
          s_B[t * BLD + j] = xc[t];
          s_B[(TMAX + t) * BLD + j] = m;
        }
      }
    } else {
      // Prefill loop: the solve sits on every chunk's critical path, so the
      // coefficients come from the lanes that formed them by readlane
      // (scalar operands), not one LDS read each (2.1 against 3.0 us per
      // chunk).  Every lane runs the substitution (lanes past TMAX form zero
      // columns); lanes j < TMAX store theirs.
      auto coef = [&](const float* r, int t, int a) {
        const int e = t * TMAX + a;
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r[e / 64]), e % 64));
      };
      const int j = lane;
      float xc[TMAX];
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        float v = (t == j) ? 1.f : 0.f;
#pragma unroll
        for (int a = 0; a < t; ++a) v = fmaf(-coef(cav, t, a), xc[a], v);
        xc[t] = (t < T && j < T) ? v : 0.f;
      }
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        float m = 0.f;
#pragma unroll
        for (int a = 0; a <= t; ++a) m = fmaf(coef(cov, t, a), xc[a], m);
        if (j < TMAX) {
          s_B[t * BLD + j] = xc[t];
          s_B[(TMAX + t) * BLD + j] = m;
        }
      }
    }
  } else {
    if constexpr (PF) {
      load_state();  // the first chunk queues the state first; later ones hold it
#pragma unroll 1
      for (int j = wave; j < PPL; j += NW) {
        typename PR::raw xr[XR];
        float w0[KM], w1[KM];
        load_pair(j, xr, w0, w1);
        conv_pair(j, xr, w0, w1);
      }
      __syncthreads();  // (B0')
    } else {
      __syncthreads();  // (B0)
    }
    if constexpr (VR) {
      // the per-key replay weights, off wave 0's path: wave 1 takes channels
      // lane and lane + 64 of the previous tape's gates g_{j,c}, j < pn
      static_assert(NW >= 2, "needs a second wave");
      if (wave == 1) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float gk[PM];
#pragma unroll
          for (int j = 0; j < PM; ++j) {
            const float gv = p.ptg[((lb * p.pT + (j < pn ? j : 0)) * p.Hv + hv) * DK + lane + 64 * h];
            gk[j] = j < pn ? gv : 1.f;
          }
          float w = 1.f;  // suffix product over j > i
#pragma unroll
          for (int i = PM - 1; i >= 0; --i) {
            s_pwk[i * DK + lane + 64 * h] = i < pn ? w : 0.f;
            w *= gk[i];
          }
          s_pgk[lane + 64 * h] = w;
        }
      }
    }
    if constexpr (PF && VG) {
      __syncthreads();  // (B_w0)
      walk_share(4 * wave + gq);
      __syncthreads();  // (B_w1)
    }
    if constexpr (!PF) load_state();
    if constexpr (PFX) {
      // The last wave (no conv share) fetches the next chunk's raw rows
      // while wave 0 solves, before its replay operands (fewer live
      // registers): x rows c0' - (K - 1) .. of chunk c' = ch + 1,
      // clamped at its end as in load_pair.  This chunk's conv has read
      // s_raw before (B0'); the next one reads it after the chunk barrier.
      if (wave == NW - 1 && ch + 1 < nch) {
        const int c0n = (ch + 1) * TMAX;
        const int nrn = K - 1 + (p0.T - c0n < TMAX ? p0.T - c0n : TMAX);
        const TIn* xb = static_cast<const TIn*>(p0.x) + lb * p0.x_ld;
#pragma unroll 1
        for (int pr = lane; pr < NPAIR; pr += 64) {
          const int chn = chan(2 * pr);
          typename PR::raw v[XR];
#pragma unroll
          for (int r = 0; r < XR; ++r) {
            const int rr = r < nrn ? r : nrn - 1;
            v[r] = PR::load(xb + static_cast<size_t>(c0n - (K - 1) + rr) * p0.C + chn);
          }
#pragma unroll
          for (int r = 0; r < XR; ++r) s_raw[r * NPAIR + pr] = v[r];
        }
      }
    }
    load_tape();
  }
  __syncthreads();  // (B1) prologue results in LDS
  if (wave == 0) {
    load_state();
    load_tape();
  }
  if constexpr (RP) {
    // S <- gamma S + sum_i w_i u_i k_i^T on this wave's tiles, as transposed
    // 16x16 tiles on fp32 MFMA: D[j][r] = sum_i k_i[16m + j] (w_i u_i)[r],
    // whose lane (c16, kk) holds exactly the sreg[.][m] element of row c16,
    // columns 16m + 4kk .. +3.  The rolled state is written back in place.
    if (pn > 0) {
      const float gam = s_pgam;
      float wv[PM / 4];
#pragma unroll
      for (int st = 0; st < PM / 4; ++st) wv[st] = VR ? 1.f : s_pw[4 * st + kk];
      if constexpr (VR) {
        // per-key weights go on the k operand: k_i[c] w_{i,c}
#pragma unroll
        for (int st = 0; st < PM / 4; ++st)
          if (4 * st < pn) {
#pragma unroll
            for (int m = 0; m < DK / 16; ++m) kt[st][m] *= s_pwk[(4 * st + kk) * DK + 16 * m + c16];
          }
      }
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const int tile = wave + tt * NW;
        float* const wp = S_live + (tile * 16 + c16) * DK + 4 * kk;
        float bu[PM / 4];
#pragma unroll
        for (int st = 0; st < PM / 4; ++st) bu[st] = 4 * st + kk < pn ? ut[tt][st] * wv[st] : 0.f;
#pragma unroll
        for (int m = 0; m < DK / 16; ++m) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int st = 0; st < PM / 4; ++st)
            if (4 * st < pn) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kt[st][m], bu[st], acc, 0, 0, 0);
          if constexpr (VR)  // columns 16m + 4kk .. +3 decay by their own gamma
            sreg[tt][m] = sreg[tt][m] * *reinterpret_cast<const floatx4*>(s_pgk + 16 * m + 4 * kk) + acc;
          else
            sreg[tt][m] = sreg[tt][m] * gam + acc;
          if constexpr (!PF) *reinterpret_cast<floatx4*>(wp + 16 * m) = sreg[tt][m];
        }
      }
    }
  }

  // this lane's node in each column block: k rows then q rows
  float cnode[NCB], cbv[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int n = cb * 16 + c16;
    const int t = n < TMAX ? n : n - TMAX;
    cnode[cb] = n < TMAX ? s_ck[t] : s_cq[t];
    cbv[cb] = s_cb[t];
  }
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int tile = wave + tt * NW;
    // S0 [K;Q]^T: A = this 16-row tile (registers), B = raw k/q rows.
    floatx4 acc1[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc1[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      bf16x8 ahi, alo;
      // 16-token chunks sit at the register limit: the one-value-at-a-time
      // split keeps them from spilling (the prefill loop, which spills a
      // little either way, spills less with the paired split)
      if constexpr (TMAX > 8 && !PF)
        split_bf16x8(sreg[tt][2 * s], sreg[tt][2 * s + 1], ahi, alo);
      else
        split_bf16x8_pk(sreg[tt][2 * s], sreg[tt][2 * s + 1], ahi, alo);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const unsigned char* br = s_kq + (cb * 16 + c16) * KQS + kk * 32 + s * 128;
        const bf16x8 bhi = *reinterpret_cast<const bf16x8*>(br);
        const bf16x8 blo = *reinterpret_cast<const bf16x8*>(br + 16);
        acc1[cb] = mfma_bf16x3(ahi, alo, bhi, blo, acc1[cb]);
      }
    }
    // RHS_t[i] = b_t v_t[i] - (b_t gamma_t r_t) (S0 k_t)[i], in place of v.
    // Only this wave touches its tile's rows, and a wave's LDS accesses
    // execute in order, so no workgroup barrier is needed around it.
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int n = cb * 16 + c16;
      if (n < TMAX) {
        float* col = s_rhs + (tile * 16 + 4 * kk) * RT_LD + n;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          col[r * RT_LD] = cbv[cb] * col[r * RT_LD] - cnode[cb] * acc1[cb][r];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // RHS^T [Ti; M2]^T on fp32 MFMA: k columns get u, q columns M2 RHS.
    floatx4 acc2[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc2[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < TMAX / 4; ++st) {
      const float a_op = s_rhs[(tile * 16 + c16) * RT_LD + 4 * st + kk];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const float b_op = s_B[(cb * 16 + c16) * BLD + 4 * st + kk];
        acc2[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_op, b_op, acc2[cb], 0, 0, 0);
      }
    }
    const int i0 = tile * 16 + 4 * kk;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int n = cb * 16 + c16;
      const bool isk = n < TMAX;
      const int t = isk ? n : n - TMAX;
      if (t < T) {
        const size_t oi = isk ? ((lb * T + t) * p.Hv + hv) * DV + i0
                              : lb * p.o_ld + (static_cast<size_t>(t) * p.Hv + hv) * DV + i0;
        floatx4 val = acc2[cb];
        if (!isk) val += cnode[cb] * acc1[cb];
        __builtin_nontemporal_store(val, reinterpret_cast<floatx4*>((isk ? p.tu : p.o) + oi));
      }
    }
  }
  if constexpr (PF) {
    // this chunk's tape stores are visible to every wave of the workgroup
    // (one CU: no cache write-back needed) and its LDS reads are done before
    // the next chunk reads the tape and overwrites LDS
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  if (!PF || ch + 1 >= nch) break;
  }  // chunks

  if constexpr (PF) {
    // Fold the last chunk (every token kept) into the state and store it.
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c16 = lane & 15;
    const int kk = lane >> 4;
    const int cl = nch - 1;
    const int Tl = p0.T - cl * TMAX;
    const bool odd = cl & 1;
    const float* tu = odd ? p0.ptu : p0.tu;
    const float* tk = odd ? p0.ptk : p0.tk;
    const float* tg = odd ? p0.ptg : p0.tg;
    const size_t base = lb * Tl;
    if constexpr (VG) {
      // per-key weights of the last chunk, as in the chunk replays
      if (wave == 1) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float gk[TMAX];
#pragma unroll
          for (int j = 0; j < TMAX; ++j) {
            const float gv = tg[((base + (j < Tl ? j : 0)) * p0.Hv + hv) * DK + lane + 64 * h];
            gk[j] = j < Tl ? gv : 1.f;
          }
          float wk = 1.f;
#pragma unroll
          for (int i = TMAX - 1; i >= 0; --i) {
            s_pwk[i * DK + lane + 64 * h] = i < Tl ? wk : 0.f;
            wk *= gk[i];
          }
          s_pgk[lane + 64 * h] = wk;
        }
      }
      __syncthreads();
    }
    const float gl = !VG && lane < Tl ? tg[(base + lane) * p0.Hv + hv] : 1.f;
    float w = 1.f, gam = 1.f;  // w_lane = prod_{lane<j<Tl} g_j, gam = prod_j g_j
#pragma unroll
    for (int j = 0; j < TMAX; ++j) {
      const float gj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), j));
      gam *= gj;
      if (j > lane) w *= gj;
    }
    float kt[TMAX / 4][DK / 16];
    float bw[TMAX / 4];
#pragma unroll
    for (int st = 0; st < TMAX / 4; ++st) {
      const int i = 4 * st + kk;
      const size_t ii = base + (i < Tl ? i : 0);
      const float* kr = tk + (ii * p0.Hv + hv) * DK + c16;  // per-v-head copy
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
        kt[st][m] = kr[16 * m] * (VG ? s_pwk[i * DK + 16 * m + c16] : 1.f);
      const float wi = __shfl(w, i, kWave);
      bw[st] = i < Tl ? (VG ? 1.f : wi) : 0.f;
    }
    float* const S_dst = p0.S_out + (lb * p0.Hv + hv) * static_cast<size_t>(DV * DK);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int tile = wave + tt * NW;
      float bu[TMAX / 4];
#pragma unroll
      for (int st = 0; st < TMAX / 4; ++st) {
        const int i = 4 * st + kk;
        const size_t ii = base + (i < Tl ? i : 0);
        bu[st] = tu[(ii * p0.Hv + hv) * DV + tile * 16 + c16] * bw[st];
      }
      float* const wp = S_dst + (tile * 16 + c16) * DK + 4 * kk;
#pragma unroll
      for (int m = 0; m < DK / 16; ++m) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < TMAX / 4; ++st)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kt[st][m], bu[st], acc, 0, 0, 0);
        if constexpr (VG)
          *reinterpret_cast<floatx4*>(wp + 16 * m) =
              sreg_pf[tt][m] * *reinterpret_cast<const floatx4*>(s_pgk + 16 * m + 4 * kk) + acc;
        else
          *reinterpret_cast<floatx4*>(wp + 16 * m) = sreg_pf[tt][m] * gam + acc;
      }
    }
  }
}

template <int DK, int DV, typename TIn, bool RP>
hipError_t launch_cr(const VerifyArgs& a, const dim3& gd, hipStream_t s) {
  constexpr int NT = chain_threads<DV>();
  if (a.T <= 8) {
    if (a.K == 4) hipLaunchKernelGGL((k_verify_chain<DK, DV, 8, 4, TIn, RP>), gd, dim3(NT), 0, s, a);
    else hipLaunchKernelGGL((k_verify_chain<DK, DV, 8, 0, TIn, RP>), gd, dim3(NT), 0, s, a);
  } else {
    if (a.K == 4) hipLaunchKernelGGL((k_verify_chain<DK, DV, 16, 4, TIn, RP>), gd, dim3(NT), 0, s, a);
    else hipLaunchKernelGGL((k_verify_chain<DK, DV, 16, 0, TIn, RP>), gd, dim3(NT), 0, s, a);
  }
  return hipGetLastError();
}

template <int DK, int DV, typename TIn>
hipError_t launch_c(const VerifyArgs& a, hipStream_t s) {
  const int G = a.Hv / a.Hk;
  const int n_units = a.L * a.B * a.Hk;
  const long long grid = static_cast<long long>((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * G;
  if (grid > 0x7fffffffLL || a.T > 16) return hipErrorInvalidValue;
  const dim3 gd(static_cast<int>(grid));
  if (a.prev_n_keep || a.prev_n_all > 0) {
    if (a.pT > 16 || a.prev_n_all > a.pT || !a.S_out || !a.ptu || !a.ptk || !a.ptg)
      return hipErrorInvalidValue;
    return launch_cr<DK, DV, TIn, true>(a, gd, s);
  }
  return launch_cr<DK, DV, TIn, false>(a, gd, s);
}

template <typename TIn>
hipError_t launch_cd(const VerifyArgs& a, int dk, int dv, hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 32: return launch_c<32, 32, TIn>(a, s);
    case 64: return launch_c<64, 64, TIn>(a, s);
    case 128: return launch_c<128, 128, TIn>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_verify_chain(const VerifyArgs& a, int dk, int dv, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_cd<uint16_t>(a, dk, dv, s) : launch_cd<float>(a, dk, dv, s);
}

hipError_t launch_verify_chain_pf(const VerifyArgs& a, int dk, int dv, int dtype, hipStream_t s) {
  const int G = a.Hv / a.Hk;
  const int n_units = a.L * a.B * a.Hk;
  const long long grid = static_cast<long long>((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * G;
  if (grid > 0x7fffffffLL || dk != 128 || dv != 128 || a.T < 1 || a.K > 16 || a.prev_n_keep ||
      !a.S_out || !a.tu || !a.tk || !a.tg || !a.ptu || !a.ptk || !a.ptg)
    return hipErrorInvalidValue;
  const dim3 gd(static_cast<int>(grid)), bd(chain_threads<128>());
  if (dtype == 1) {
    if (a.K == 4) hipLaunchKernelGGL((k_verify_chain<128, 128, 16, 4, uint16_t, true, false, true>), gd, bd, 0, s, a);
    else hipLaunchKernelGGL((k_verify_chain<128, 128, 16, 0, uint16_t, true, false, true>), gd, bd, 0, s, a);
  } else {
    if (a.K == 4) hipLaunchKernelGGL((k_verify_chain<128, 128, 16, 4, float, true, false, true>), gd, bd, 0, s, a);
    else hipLaunchKernelGGL((k_verify_chain<128, 128, 16, 0, float, true, false, true>), gd, bd, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_verify_chain_vg_pf(const VerifyArgs& a, hipStream_t s) {
  const int G = a.Hv / a.Hk;
  const int n_units = a.L * a.B * a.Hk;
  const long long grid = static_cast<long long>((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * G;
  if (grid > 0x7fffffffLL || a.T < 1 || a.K > 16 || a.prev_n_keep || !a.S_out || !a.tu ||
      !a.tk || !a.tg || !a.ptu || !a.ptk || !a.ptg)
    return hipErrorInvalidValue;
  const dim3 gd(static_cast<int>(grid)), bd(chain_threads<128>());
  if (a.K == 4) hipLaunchKernelGGL((k_verify_chain<128, 128, 16, 4, uint16_t, true, true, true>), gd, bd, 0, s, a);
  else hipLaunchKernelGGL((k_verify_chain<128, 128, 16, 0, uint16_t, true, true, true>), gd, bd, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_verify_chain_vg(const VerifyArgs& a, hipStream_t s) {
  const int G = a.Hv / a.Hk;
  const int n_units = a.L * a.B * a.Hk;
  const long long grid = static_cast<long long>((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * G;
  if (grid > 0x7fffffffLL || a.T > 16) return hipErrorInvalidValue;
  const dim3 gd(static_cast<int>(grid)), bd(chain_threads<128>());
  if (a.prev_n_keep || a.prev_n_all > 0) {
    if (a.pT > 16 || a.prev_n_all > a.pT || !a.S_out || !a.ptu || !a.ptk || !a.ptg)
      return hipErrorInvalidValue;
    if (a.T <= 8) {
      if (a.K == 4) hipLaunchKernelGGL((k_verify_chain<128, 128, 8, 4, uint16_t, true, true>), gd, bd, 0, s, a);
      else hipLaunchKernelGGL((k_verify_chain<128, 128, 8, 0, uint16_t, true, true>), gd, bd, 0, s, a);
    } else {
      if (a.K == 4) hipLaunchKernelGGL((k_verify_chain<128, 128, 16, 4, uint16_t, true, true>), gd, bd, 0, s, a);
      else hipLaunchKernelGGL((k_verify_chain<128, 128, 16, 0, uint16_t, true, true>), gd, bd, 0, s, a);
    }
    return hipGetLastError();
  }
  if (a.T <= 8) {
    if (a.K == 4) hipLaunchKernelGGL((k_verify_chain<128, 128, 8, 4, uint16_t, false, true>), gd, bd, 0, s, a);
    else hipLaunchKernelGGL((k_verify_chain<128, 128, 8, 0, uint16_t, false, true>), gd, bd, 0, s, a);
  } else {
    if (a.K == 4) hipLaunchKernelGGL((k_verify_chain<128, 128, 16, 4, uint16_t, false, true>), gd, bd, 0, s, a);
    else hipLaunchKernelGGL((k_verify_chain<128, 128, 16, 0, uint16_t, false, true>), gd, bd, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace gdn
