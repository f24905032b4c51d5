// k_verify_tree.hip -- verify of a draft tree of up to 64 nodes through one GDN
// layer (128-dim heads, bf16 inputs), for gfx950.
//
// Per node v with parent p (p = -1: the committed state S0), the gated delta
// rule of the GDN page (s2.1) steps from the parent's state:
//   S_v = a_v S_p + u_v k_v^T,  u_v = b_v (v_v - a_v S_p k_v),  o_v = S_v q_v,
// which is how a draft tree is verified through the recurrent state in one
// pass (GDN page s8, tree-aware verify).  Unrolled along the root path of each
// node (path(t) = its ancestors and itself, in depth order p_0 .. p_{d-1} = t),
// with Gamma[t,i] the product of a over the path strictly below i up to t:
//   (I + A) U = RHS,  A[t,i] = b_t Gamma[t,i] k_t.k_i   (i a proper ancestor)
//   RHS_t = b_t (v_t - gamma_t S0 k_t),  gamma_t = prod of a over path(t)
//   o_t = gamma_t S0 q_t + sum_{i in path(t)} Oc[t,i] u_i,  Oc[t,i] = Gamma[t,i] q_t.k_i
// With Ti = (I + A)^-1 and M2 = Oc Ti:  U = Ti RHS,  O = diag(gamma) Q S0^T + M2 RHS.
// Ti and M2 are supported on ancestor-or-self pairs, and row t of Ti depends
// only on the entries of A among the nodes of path(t): each node solves its
// own row (backward substitution along its path), with no level-by-level
// barriers.  A, Oc, Ti and M2 live in packed rows (row t holds one value per
// node of path(t), slot = depth - 1), at most T(T+1)/2 values each.
//
// One workgroup of eight waves per (layer, seq, v-head) -- or, with two
// v-heads per k-head and conv width 4, per (layer, seq, k-head) running both
// v-heads: their q/k conv, norms, pre-split operand and Gram are the same, so
// they are done once and only the gate-dependent solve and the state
// products repeat per head.  Wave w owns rows 16w .. 16w+15 of each head's
// S0 (registers, MFMA A operand).  Phases:
//   loads: parents, gates, the raw conv rows (staged in LDS), conv weights;
//   wave 0: node depths, ancestor masks, conv windows, path products, packed
//     row offsets (one lane per node, wave-level scan);
//   conv + SiLU: one 16-lane group per (node, q/k/v segment), 8 channels per
//     lane; q and k rows are L2-normalised with a 16-lane reduction, written
//     as pre-split bf16 hi/lo MFMA operands, and k goes to the tape;
//   Gram [K;Q] K^T on bf16x3 MFMA, keeping only ancestor-or-self entries;
//   the packed Ti and M2 rows are solved (trees of depth <= 8: in registers
//   on waves 2 and 3, one head each; deeper trees: on wave 0) while the
//   other waves run S0 [K;Q]^T (bf16x3 MFMA) and form RHS in LDS;
//   [Ti; M2] is expanded to a dense pre-split operand in the space of K/Q;
//   RHS [Ti; M2]^T (bf16x3 MFMA); u and o are stored from registers.
// With two heads the second head's S0 [K;Q]^T runs right after the first's
// (K/Q are still in LDS), its v rows wait in registers until the first head
// has finished with the V space, and its packed rows (solved beside the
// first head's, or on wave 0 during the first head's second product for
// trees deeper than 8) are written once the first head's are expanded.
// S0 and the conv window are never written (they stay the snapshot), except
// by the replay form.
//
// Forms (template flags): RP first folds the previous round's accepted path
// into S (the rank-n tape replay on fp32 MFMA, written back in place); VG
// takes the decay gate per key channel (one head per workgroup: a path walk
// forms the A and Oc coefficients from forward gate products, the operand
// rows carry gamma, and the replay puts per-channel path weights, formed
// backwards along the path in registers, on its k operand).

#include "gdn_common.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

constexpr int TR_D = 128;       // head dimension (Dk = Dv)
constexpr int TR_T = 64;        // nodes per tree (padded)
constexpr int TR_NT = 512;      // eight waves
constexpr int TR_KQS = 528;     // bytes per pre-split [K;Q] row: 128 x (hi, lo) + 16 pad
constexpr int TR_B2S = 272;     // bytes per pre-split [Ti;M2] row: 64 x (hi, lo) + 16 pad
constexpr int TR_VLD = 68;      // floats per V / RHS row ([row of S][node])

// Position of node t in V / RHS row i: 8-node groups are permuted by the row's
// 8-row block, so the transposing writes of the conv spread over the banks
// while each group of 8 nodes stays contiguous for float4 reads.
__device__ __forceinline__ int vsw(int i) { return ((i >> 3) & 7) << 3; }
constexpr int TR_PK = TR_T * (TR_T + 1) / 2;  // packed triangle capacity

__device__ __forceinline__ float silu_t(float y) {
  return y * __builtin_amdgcn_rcpf(1.f + __expf(-y));
}

// x moved across lanes by the DPP control CTRL into the rows of ROW_MASK;
// lanes without a source (and rows outside the mask) get 1.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}

// Sum over aligned groups of 16 lanes (DPP; every lane gets its group's sum).
__device__ __forceinline__ float sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// Pack four fp32 values as bf16 high parts and bf16 residuals (8 bytes each).
__device__ __forceinline__ void split4(const float* y, uint2& hi, uint2& lo) {
  split_pair(y[0], y[1], hi.x, lo.x);
  split_pair(y[2], y[3], hi.y, lo.y);
}

template <int KM, int NH>
struct TreeLds {
  static constexpr int ROWB = (2 + NH) * TR_D * 2;  // raw staging bytes per row (q | k | v rows)
  static constexpr int XR = TR_T + KM - 1;  // raw rows: old window, then nodes
  static constexpr int STAGE = XR * ROWB;
  static constexpr int VBYTES = TR_D * TR_VLD * 4;
  static constexpr int PKBYTES = 4 * TR_PK * 4;  // KK, QK, Ti, M2
  static constexpr int R2 = STAGE > VBYTES + PKBYTES ? STAGE : VBYTES + PKBYTES;
  static constexpr int R1 = 2 * TR_T * TR_KQS;
};

// One (layer, seq, k-head or v-head) unit; bid plays the role of the block
// index.  All threads leave together.
template <int KC, bool RP, int NH, bool VG>
__device__ __forceinline__ void tree_unit(const VerifyArgs& p, const int bid) {
  static_assert(!VG || NH == 1, "the per-key-channel gate runs one head");
  constexpr int KM = KC > 0 ? KC : 8;
  using LY = TreeLds<KM, NH>;
  constexpr int XR = LY::XR;
  constexpr int ROWB = LY::ROWB;
  constexpr int NSEG = 2 + NH;  // conv segments: q, k, then v of each head
  static_assert(2 * TR_T * TR_B2S <= LY::R1, "[Ti;M2] operand fits in the K/Q space");
  static_assert(LY::R1 + LY::R2 + NSEG * TR_D * KM * 4 + TR_T * (40 + 12 * NH + 4 * KM) <= 160 * 1024,
                "LDS budget");

  __shared__ __align__(16) unsigned char s_r1[LY::R1];  // pre-split [K;Q], later [Ti;M2]
  __shared__ __align__(16) unsigned char s_r2[LY::R2];  // raw staging, later V/RHS + packed
  // conv weights [segment][e][li][tap] for channel 8 li + e of the segment:
  // the conv's 16-lane groups read them as consecutive 16-byte chunks
  __shared__ __align__(16) float s_w[NSEG * TR_D * KM];
  __shared__ unsigned long long s_anc[TR_T];            // proper-ancestor masks
  __shared__ int s_par[TR_T], s_dep[TR_T], s_off[TR_T];
  __shared__ __align__(16) int s_widx[TR_T * KM];       // conv window: staging byte offsets
  __shared__ float s_ga[NH * TR_T], s_gb[NH * TR_T], s_gam[NH * TR_T];  // per head
  __shared__ int s_bad, s_maxd;
  // previous round's accepted path (replay variant): tape entry of step i,
  // w_i = prod_{i<j<pn} g_j (zero for i >= pn), gamma = prod_{j<pn} g_j
  __shared__ int s_ppath[RP ? TR_T : 1];
  __shared__ float s_pw[RP ? NH * TR_T : 1];
  __shared__ float s_pgam[NH];
  __shared__ int s_pbad;

  float* s_v = reinterpret_cast<float*>(s_r2);            // [row of S][node]
  float* s_KK = s_v + TR_D * TR_VLD;                      // packed rows
  float* s_QK = s_KK + TR_PK;
  float* s_TI = s_QK + TR_PK;
  float* s_M2 = s_TI + TR_PK;

  // an opaque copy of the lane index per unit, so that the compiler
  // recomputes lane-dependent addresses inside the unit loop instead of
  // keeping them live across it
  int tid_l = threadIdx.x;
  asm volatile("" : "+v"(tid_l));
  const int tid = tid_l;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int kk = lane >> 4;

  const int G = p.Hv / p.Hk;
  const int n_units = p.L * p.B * p.Hk;
  const UnitSub us = xcd_unit_sub(bid, G / NH);
  if (us.unit >= n_units) return;
  const int hk = us.unit % p.Hk;
  const size_t lb = us.unit / p.Hk;  // l * B + b
  const int bb = static_cast<int>(lb % p.B);
  const int l = static_cast<int>(lb / p.B);
  const int g = us.sub * NH;
  const int hv = hk * G + g;  // first v-head of this workgroup (heads hv .. hv + NH - 1)
  const int T = p.T;
  const int K = KC > 0 ? KC : p.K;
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const uint16_t* cs = static_cast<const uint16_t*>(p.conv_state);
  // accepted length of the previous round (replay variant)
  int pn = 0;
  if constexpr (RP) {
    const int v = p.prev_n_keep[bb];
    pn = (v >= 0 && v <= p.pT) ? v : 0;
    if (pn != v && tid == 0 && p.dev_err && l == 0 && hk == 0 && g == 0)
      atomicOr(p.dev_err, GDN_DEV_ERR_N_KEEP);
  }

  // ------------------------------------------------------------------ loads --
  // Every load is unconditional from a clamped, valid address.
  const int tq = lane < T ? lane : 0;
  const int par_raw = p.parent[static_cast<size_t>(bb) * T + tq];
  const size_t gi = (lb * T + tq) * p.Hv + hv;
  float ga_ld[NH], gb_ld[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    // per-key-channel gates enter through the operands instead (below)
    ga_ld[h] = VG ? 1.f : ld_in(static_cast<const uint16_t*>(p.a), gi + h);
    gb_ld[h] = ld_in(static_cast<const uint16_t*>(p.b), gi + h);
  }
  // per-key-channel gates of the head, [node][channel]: thread tid holds node
  // tid / 8, channels 16 (tid % 8) .. +15
  u32x4 avr[VG ? 2 : 1];
  if constexpr (VG) {
    const int tn = tid / 8;
    const uint16_t* ap = static_cast<const uint16_t*>(p.a) +
                         ((lb * T + (tn < T ? tn : 0)) * p.Hv + hv) * TR_D + 16 * (tid % 8);
    avr[0] = *reinterpret_cast<const u32x4*>(ap);
    avr[1] = *reinterpret_cast<const u32x4*>(ap + 8);
  }
  // local channel c in [q | k | v-rows] -> qkv channel
  auto chan = [&](int c) {
    return c < TR_D ? hk * TR_D + c
                    : (c < 2 * TR_D ? p.Hk * TR_D + hk * TR_D + (c - TR_D)
                                    : 2 * p.Hk * TR_D + hv * TR_D + (c - 2 * TR_D));
  };
  constexpr int CPR = ROWB / 16;                        // 16-byte chunks per raw row
  constexpr int NRAW = (XR * CPR + TR_NT - 1) / TR_NT;  // per thread
  const int nrows = K - 1 + T;
  const uint16_t* xcol = x + lb * T * p.C;
  const uint16_t* ccol = cs + lb * (K - 1) * p.C;
  u32x4 raw[NRAW];
#pragma unroll
  for (int q = 0; q < NRAW; ++q) {
    const int e = tid + q * TR_NT;
    const int row = e / CPR, chunk = e % CPR;
    const int rr = row < nrows ? row : nrows - 1;
    const uint16_t* base = rr < K - 1 ? ccol + static_cast<size_t>(rr) * p.C
                                      : xcol + static_cast<size_t>(rr - (K - 1)) * p.C;
    raw[q] = *reinterpret_cast<const u32x4*>(base + chan(chunk * 8));
  }
  // conv weights of the 384 channels, zero beyond the kernel width
  const float* cw = p.conv_w + static_cast<size_t>(l) * p.C * K;
  constexpr int NWL = (NSEG * TR_D * KM + TR_NT - 1) / TR_NT;
  float wv[NWL];
#pragma unroll
  for (int q = 0; q < NWL; ++q) {
    const int e = tid + q * TR_NT;
    const int c = e / KM, j = e % KM;
    const bool ok = e < NSEG * TR_D * KM && j < K;
    const float v = cw[static_cast<size_t>(chan(ok ? c : 0)) * K + (ok ? j : 0)];
    wv[q] = ok ? v : 0.f;
  }

  // --------------------------------------------- node structure (wave 0) --
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (wave == 0) {
    const int t = lane;
    int pv = -1;
    if (t < T) {
      pv = par_raw;
      if (pv < -1 || pv >= t) {
        s_bad = 1;
        pv = -1;
      }
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        s_ga[h * TR_T + t] = ga_ld[h];
        s_gb[h * TR_T + t] = gb_ld[h];
        if (!VG) p.tg[(lb * T + t) * p.Hv + hv + h] = ga_ld[h];
      }
    } else {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        s_ga[h * TR_T + t] = 1.f;
        s_gb[h * TR_T + t] = 0.f;
      }
    }
    s_par[t] = pv;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ancestors, depth, path product of a, conv window (node, then upward)
    unsigned long long m = 0ull;
    int d = 0;
    float gm[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) gm[h] = 1.f;
    if (t < T) {
#pragma unroll
      for (int h = 0; h < NH; ++h) gm[h] = s_ga[h * TR_T + t];
      d = 1;
      for (int c = s_par[t]; c >= 0; c = s_par[c]) {
        m |= 1ull << c;
#pragma unroll
        for (int h = 0; h < NH; ++h) gm[h] *= s_ga[h * TR_T + c];
        ++d;
      }
    }
    s_anc[t] = m;
    s_dep[t] = d;
#pragma unroll
    for (int h = 0; h < NH; ++h) s_gam[h * TR_T + t] = gm[h];
    {
      int cur = t < T ? t : -1, old = 0;
#pragma unroll
      for (int j = KM - 1; j >= 0; --j) {
        int w = 0;
        if (j < K) {
          if (cur >= 0) {
            w = cur;
            cur = s_par[cur];
          } else {
            w = --old;
          }
        }
        s_widx[t * KM + j] = (w + K - 1) * ROWB;
      }
    }
    // packed row offsets: exclusive prefix sum of depths over nodes
    int incl = d;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    s_off[t] = incl - d;
    int md = d;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) md = max(md, __shfl_xor(md, o, 64));
    if (lane == 0) s_maxd = md;
  }
  if constexpr (RP) {
    // wave 1: the previous accepted path, validated, and its gate products
    if (wave == 1) {
      int pp = lane;
      bool bad = false;
      if (lane < pn) {
        if (p.prev_path) pp = p.prev_path[static_cast<size_t>(bb) * p.pT + lane];
        bad = pp < 0 || pp >= p.pT;
      }
      pp = lane < pn && !bad ? pp : 0;
#pragma unroll
      for (int h = 0; h < (VG ? 0 : NH); ++h) {  // (per-key weights: formed in the replay)
        const float gv = lane < pn ? p.ptg[(lb * p.pT + pp) * p.Hv + hv + h] : 1.f;
        float x_s = gv;  // inclusive suffix product prod_{j >= lane} g_j
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const float y = __shfl_down(x_s, o, 64);
          if (lane + o < 64) x_s *= y;
        }
        float w = __shfl_down(x_s, 1, 64);
        if (lane == 63) w = 1.f;
        s_pw[h * TR_T + lane] = lane < pn ? w : 0.f;
        if (lane == 0) s_pgam[h] = x_s;
      }
      s_ppath[lane] = pp;
      const unsigned long long anybad = __ballot(bad);
      if (lane == 0) s_pbad = anybad != 0ull;
    }
  }
  // raw rows and weights into LDS
  u32x4* s_stage = reinterpret_cast<u32x4*>(s_r2);
#pragma unroll
  for (int q = 0; q < NRAW; ++q) {
    const int e = tid + q * TR_NT;
    if (e < XR * CPR) s_stage[e] = raw[q];
  }
#pragma unroll
  for (int q = 0; q < NWL; ++q) {
    const int e = tid + q * TR_NT;
    if (e < NSEG * TR_D * KM) {
      const int c = e / KM, j = e % KM;  // loaded as [channel][tap]
      const int sg = c / TR_D, cc = c % TR_D;
      s_w[((sg * 8 + cc % 8) * 16 + cc / 8) * KM + j] = wv[q];
    }
  }
  __syncthreads();  // (B_a) staging, weights, node structure
  if constexpr (RP) {
    if (s_pbad) {
      if (tid == 0 && p.dev_err && l == 0 && hk == 0 && g == 0) atomicOr(p.dev_err, GDN_DEV_ERR_PATH);
      pn = 0;
    }
  }

  // Replay operands of the first 4 PRE steps, straight from the previous tape
  // into registers: lane (c16, kk) takes k_{p_i}[16m + c16] (A) and
  // u_{p_i}[16 wave + c16] (B) for i = 4 st + kk; longer paths load the
  // remaining steps as they go.  Steps with 4 st >= pn are skipped (pn is
  // uniform).
  constexpr int PRE = NH > 1 ? 2 : 4;  // groups of four steps preloaded
  float kt[RP ? PRE : 1][RP ? TR_D / 16 : 1];
  float ut[NH][RP ? PRE : 1];
  auto load_step = [&](int st, float* ka, float* ua) __attribute__((always_inline)) {
    const int i = 4 * st + kk;
    const size_t e = lb * p.pT + s_ppath[i < pn ? i : 0];
    const float* kr = p.ptk + (e * p.Hk + hk) * TR_D + c16;
#pragma unroll
    for (int m = 0; m < TR_D / 16; ++m) ka[m] = kr[16 * m];
#pragma unroll
    for (int h = 0; h < NH; ++h) ua[h] = p.ptu[(e * p.Hv + hv + h) * TR_D + wave * 16 + c16];
  };
  auto preload_steps = [&]() {
    if constexpr (RP) {
#pragma unroll
      for (int st = 0; st < PRE; ++st) {
        if (4 * st < pn) {
          float ua[NH];
          load_step(st, kt[st], ua);
#pragma unroll
          for (int h = 0; h < NH; ++h) ut[h][st] = ua[h];
        }
      }
    }
  };
  // one head: the operands load under the conv; two heads: after it (held
  // through the longer conv they would spill)
  if constexpr (NH == 1) preload_steps();
  // state tiles of this wave, one per head
  floatx4 sreg[NH][TR_D / 16];
  const float* srow = p.S + (lb * p.Hv + hv) * static_cast<size_t>(TR_D * TR_D) +
                      static_cast<size_t>(wave * 16 + c16) * TR_D + 4 * kk;
  // S <- gamma S + sum_i w_i u_{p_i} k_{p_i}^T on this wave's tile, as
  // transposed 16x16 fp32 MFMA tiles D[j][r] = sum_i k_i[16m + j] (w_i u_i)[r]
  // (lane (c16, kk) of D holds exactly sreg[m]); the rolled tile is written
  // back in place.
  // Per-key gate: S <- S diag(gamma) + sum_i u_{p_i} (k_{p_i} o w_i)^T with
  // w_i[c] = prod_{i<j<pn} g_{p_j}[c] and gamma[c] = prod_{j<pn} g_{p_j}[c].
  // Step groups go from the last to the first; each lane keeps, for its
  // channels 16m + c16, the product R[m] of the gates of the groups already
  // done, and its step 4 st + kk takes R times the gates of the later steps
  // of its own group on the k operand.
  auto replay_vg = [&]() __attribute__((always_inline)) {
    if constexpr (RP && VG) {
      floatx4 acc[TR_D / 16];
      float R[TR_D / 16];
#pragma unroll
      for (int m = 0; m < TR_D / 16; ++m) {
        acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
        R[m] = 1.f;
      }
      auto group = [&](int st, const float* ka, float ua) __attribute__((always_inline)) {
        float gq[4][TR_D / 16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = 4 * st + q;
          const float* gr = p.ptg + ((lb * p.pT + s_ppath[j < pn ? j : 0]) * p.Hv + hv) * TR_D + c16;
#pragma unroll
          for (int m = 0; m < TR_D / 16; ++m) {
            const float gv = gr[16 * m];
            gq[q][m] = j < pn ? gv : 1.f;
          }
        }
        const int i = 4 * st + kk;
        const float bu = i < pn ? ua : 0.f;
#pragma unroll
        for (int m = 0; m < TR_D / 16; ++m) {
          float w = R[m];
#pragma unroll
          for (int q = 1; q < 4; ++q) w *= q > kk ? gq[q][m] : 1.f;
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[m] * w, bu, acc[m], 0, 0, 0);
          R[m] *= gq[0][m] * gq[1][m] * gq[2][m] * gq[3][m];
        }
      };
      const int ng = (pn + 3) / 4;
      for (int st = ng - 1; st >= PRE; --st) {
        float ka[TR_D / 16], ua[NH];
        load_step(st, ka, ua);
        group(st, ka, ua[0]);
      }
#pragma unroll
      for (int st = PRE - 1; st >= 0; --st)
        if (4 * st < pn) group(st, kt[st], ut[0][st]);
      // columns 16m + 4kk + e decay by gamma of that channel, held by lane 4kk + e
#pragma unroll
      for (int m = 0; m < TR_D / 16; ++m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gm = __shfl(R[m], 4 * kk + e, 64);
          sreg[0][m][e] = sreg[0][m][e] * gm + acc[m][e];
        }
      }
    }
  };
  auto replay = [&](int h) __attribute__((always_inline)) {
    if constexpr (RP && VG) {
      replay_vg();
    } else if constexpr (RP) {
      floatx4 acc[TR_D / 16];
#pragma unroll
      for (int m = 0; m < TR_D / 16; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < PRE; ++st) {
        if (4 * st < pn) {
          const int i = 4 * st + kk;
          const float bu = i < pn ? ut[h][st] * s_pw[h * TR_T + i] : 0.f;
#pragma unroll
          for (int m = 0; m < TR_D / 16; ++m)
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(kt[st][m], bu, acc[m], 0, 0, 0);
        }
      }
      for (int st = PRE; 4 * st < pn; ++st) {
        float ka[TR_D / 16], ua[NH];
        load_step(st, ka, ua);
        const int i = 4 * st + kk;
        const float bu = i < pn ? ua[h] * s_pw[h * TR_T + i] : 0.f;
#pragma unroll
        for (int m = 0; m < TR_D / 16; ++m)
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[m], bu, acc[m], 0, 0, 0);
      }
      const float gam = s_pgam[h];
#pragma unroll
      for (int m = 0; m < TR_D / 16; ++m) sreg[h][m] = sreg[h][m] * gam + acc[m];
    }
  };
  // the rolled tiles back to the live state
  auto store_replayed = [&]() {
    if constexpr (RP) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        float* wrow = p.S_out + (lb * p.Hv + hv + h) * static_cast<size_t>(TR_D * TR_D) +
                      static_cast<size_t>(wave * 16 + c16) * TR_D + 4 * kk;
#pragma unroll
        for (int m = 0; m < TR_D / 16; ++m) *reinterpret_cast<floatx4*>(wrow + 16 * m) = sreg[h][m];
      }
    }
  };

  if (s_bad) {
    if (tid == 0 && p.dev_err) atomicOr(p.dev_err, GDN_DEV_ERR_PARENT);
    // the previous round's replay is still owed to the state
    if (RP && pn > 0) {
      if constexpr (NH > 1) preload_steps();
#pragma unroll
      for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int m = 0; m < TR_D / 16; ++m)
          sreg[h][m] = *reinterpret_cast<const floatx4*>(srow + h * TR_D * TR_D + 16 * m);
        replay(h);
      }
      store_replayed();
    }
    return;
  }
  if (p.conv_win && l == 0 && hk == 0 && g == 0) {
    for (int e = tid; e < T * K; e += TR_NT)
      p.conv_win[static_cast<size_t>(bb) * T * K + e] = s_widx[(e / K) * KM + (e % K)] / ROWB - (K - 1);
  }

  // The state tile of this wave: lane (c16, kk) holds row 16w + c16, columns
  // 16m + 4kk .. +3, used after the conv and the Gram.  Its loads go out two
  // per conv round: issued as one burst they would stall the wave until the
  // memory pipeline had accepted them all.

  // ---------------------------------------------------------- conv + SiLU --
  // 16-lane group gr handles (segment, node) items gr + 32 r; lane li holds
  // channels 8 li .. 8 li + 7 of the segment.
  const int gr = tid >> 4, li = tid & 15;
  float vout[2 * NH][8];
#pragma unroll
  for (int r = 0; r < 2 * NSEG; ++r) {
    if (r < NH * TR_D / 32) {
      // head r / 4, columns 32 (r % 4) .. +31
      const float* sr = srow + (r / 4) * TR_D * TR_D + 32 * (r % 4);
      sreg[r / 4][2 * (r % 4)] = *reinterpret_cast<const floatx4*>(sr);
      sreg[r / 4][2 * (r % 4) + 1] = *reinterpret_cast<const floatx4*>(sr + 16);
    }
    const int item = gr + 32 * r;
    const int sg = item / TR_T;  // 0 q, 1 k, 2.. v of each head (uniform per round)
    const int t = item % TR_T;
    const int4 wa = *reinterpret_cast<const int4*>(s_widx + t * KM);
    int wi[KM];
    wi[0] = wa.x;
    if (KM > 1) wi[1 % KM] = wa.y;
    if (KM > 2) wi[2 % KM] = wa.z;
    if (KM > 3) wi[3 % KM] = wa.w;
    if constexpr (KM > 4) {
      const int4 wb = *reinterpret_cast<const int4*>(s_widx + t * KM + 4);
      wi[4 % KM] = wb.x;
      wi[5 % KM] = wb.y;
      wi[6 % KM] = wb.z;
      wi[7 % KM] = wb.w;
    }
    u32x4 xv[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      xv[j] = *reinterpret_cast<const u32x4*>(s_r2 + wi[j] + sg * 256 + li * 16);
    float y[8];
    const float* wrow = s_w + (sg * TR_D + li) * KM;  // + 16 KM per channel step e
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        const uint32_t wd = xv[j][e / 2];
        const float xe = __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16));
        acc = fmaf(wrow[e * 16 * KM + j], xe, acc);
      }
      if (p.silu) acc = silu_t(acc);
      y[e] = t < T ? acc : 0.f;
    }
    if (sg < 2) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
      ss = sum16(ss);
      const float rn = t < T ? __builtin_amdgcn_rsqf(ss + p.eps) : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= rn;
      if (sg == 1 && g == 0 && t < T) {
        floatx4* dst = reinterpret_cast<floatx4*>(p.tk + ((lb * T + t) * p.Hk + hk) * TR_D + 8 * li);
        __builtin_nontemporal_store(floatx4{y[0], y[1], y[2], y[3]}, dst);
        __builtin_nontemporal_store(floatx4{y[4], y[5], y[6], y[7]}, dst + 1);
      }
      // pre-split operand row n: element c = 8 li + e sits at 32-column step
      // c / 32, half (c % 32) / 16, lane group (c % 16) / 4, slot c % 4.
      const int n = sg == 0 ? TR_T + t : t;
      const int s = li / 4, h = (li % 4) / 2, kg = 2 * (li % 2);
      unsigned char* row = s_r1 + n * TR_KQS + s * 128 + h * 8;
      uint2 hi, lo;
      split4(y, hi, lo);
      *reinterpret_cast<uint2*>(row + kg * 32) = hi;
      *reinterpret_cast<uint2*>(row + kg * 32 + 16) = lo;
      split4(y + 4, hi, lo);
      *reinterpret_cast<uint2*>(row + (kg + 1) * 32) = hi;
      *reinterpret_cast<uint2*>(row + (kg + 1) * 32 + 16) = lo;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) vout[r - 4][e] = y[e];
    }
  }
  if constexpr (NH > 1) __builtin_amdgcn_sched_barrier(0);  // finish the conv here
  __syncthreads();  // (B_b) staging consumed
  if constexpr (NH > 1) preload_steps();
  if constexpr (VG) {
    // Per-key-channel gate: node v's parent state applied to a_v * k_v is
    // S0 (gamma_v * k_v) + sum_i u_i c_{v,i} over v's proper ancestors i, with
    // c_{v,i} = sum_c k_i[c] w_{v,i}[c] k_v[c], w_{v,i} the product of a over
    // the path nodes below i down to v and gamma_v the product over the whole
    // path; o_v = S0 (gamma_v * q_v) + sum_i u_i d_{v,i} + u_v (k_v . q_v).
    // This is the scalar algebra with A[v,i] = b_v c_{v,i}, Oc[v,i] = d_{v,i}
    // and gamma folded into the K/Q operand rows: c and d go into the packed
    // Gram rows, the gates used by the scalar path stay 1, and each node's
    // operand rows are scaled by gamma_v.
    float* s_av = s_v;  // gates [node][channel] over the V space, until the V rows
    {
      const int tn = tid / 8, c0 = 16 * (tid % 8);
      float av[16];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          av[8 * q + 2 * w] = __uint_as_float(avr[q][w] << 16);
          av[8 * q + 2 * w + 1] = __uint_as_float(avr[q][w] & 0xffff0000u);
        }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4 v4 = {av[4 * q], av[4 * q + 1], av[4 * q + 2], av[4 * q + 3]};
        *reinterpret_cast<floatx4*>(s_av + tn * TR_D + c0 + 4 * q) = v4;
        if (tn < T)
          *reinterpret_cast<floatx4*>(p.tg + ((lb * T + tn) * p.Hv + hv) * TR_D + c0 + 4 * q) = v4;
      }
    }
    // the 8 channels 8 li .. 8 li + 7 of pre-split operand row n, and back
    auto read8 = [&](int n, float* y) {
      const unsigned char* row = s_r1 + n * TR_KQS + (li / 4) * 128 + ((li % 4) / 2) * 8;
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
    auto write8 = [&](int n, const float* y) {
      unsigned char* row = s_r1 + n * TR_KQS + (li / 4) * 128 + ((li % 4) / 2) * 8;
      const int kg = 2 * (li % 2);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint2 hi, lo;
        split4(y + 4 * hf, hi, lo);
        *reinterpret_cast<uint2*>(row + (kg + hf) * 32) = hi;
        *reinterpret_cast<uint2*>(row + (kg + hf) * 32 + 16) = lo;
      }
    };
    __syncthreads();  // gates in LDS
    // the path walk: 16-lane group gr takes nodes gr and gr + 32
    float gam[2][8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int v = gr + 32 * j;
#pragma unroll
      for (int e = 0; e < 8; ++e) gam[j][e] = 0.f;
      if (v < T) {
        float kv[8], qv[8], w[8];
        read8(v, kv);
        read8(TR_T + v, qv);
        const floatx4 w0 = *reinterpret_cast<const floatx4*>(s_av + v * TR_D + 8 * li);
        const floatx4 w1 = *reinterpret_cast<const floatx4*>(s_av + v * TR_D + 8 * li + 4);
        float kq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          w[e] = e < 4 ? w0[e] : w1[e - 4];
          kq = fmaf(kv[e], qv[e], kq);
        }
        const int off = s_off[v];
        for (int i = s_par[v]; i >= 0; i = s_par[i]) {
          float ki[8];
          read8(i, ki);
          const floatx4 a0 = *reinterpret_cast<const floatx4*>(s_av + i * TR_D + 8 * li);
          const floatx4 a1 = *reinterpret_cast<const floatx4*>(s_av + i * TR_D + 8 * li + 4);
          float cc = 0.f, dd = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float kw = ki[e] * w[e];
            cc = fmaf(kw, kv[e], cc);
            dd = fmaf(kw, qv[e], dd);
            w[e] *= e < 4 ? a0[e] : a1[e - 4];
          }
          cc = sum16(cc);
          dd = sum16(dd);
          if (li == 0) {
            const int slot = s_dep[i] - 1;
            s_KK[off + slot] = cc;
            s_QK[off + slot] = dd;
          }
        }
        kq = sum16(kq);
        if (li == 0) s_QK[off + s_dep[v] - 1] = kq;
#pragma unroll
        for (int e = 0; e < 8; ++e) gam[j][e] = w[e];
      }
    }
    __syncthreads();  // every walk has read the unscaled rows and the gates
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int v = gr + 32 * j;
      if (v < T) {
        float y[8];
        read8(v, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] *= gam[j][e];
        write8(v, y);
        read8(TR_T + v, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] *= gam[j][e];
        write8(TR_T + v, y);
      }
    }
  }
  // V rows into [row of S][node] (over the staging space)
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = (gr + 32 * (4 + r)) % TR_T;
#pragma unroll
    for (int e = 0; e < 8; ++e) s_v[(8 * li + e) * TR_VLD + (t ^ vsw(8 * li))] = vout[r][e];
  }

  // -------------------------- Gram [K;Q] K^T, ancestor-or-self entries only --
  if constexpr (!VG) {
    const int rb = wave;           // 16-row block of [K;Q]
    const bool isq = rb >= 4;
    const int nb = rb % 4;         // node block of the rows
    const unsigned char* ar = s_r1 + (rb * 16 + c16) * TR_KQS + kk * 32;
    bf16x8 ahi[4], alo[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      ahi[s] = *reinterpret_cast<const bf16x8*>(ar + s * 128);
      alo[s] = *reinterpret_cast<const bf16x8*>(ar + s * 128 + 16);
    }
    unsigned long long rm[4];
    int ro[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = nb * 16 + 4 * kk + r;
      // padding rows (depth 0) take no entries
      rm[r] = tr < T ? (s_anc[tr] | (isq ? (1ull << tr) : 0ull)) : 0ull;
      ro[r] = s_off[tr];
    }
    float* dst = isq ? s_QK : s_KK;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      if (cb > nb) break;  // columns are ancestors: never above the row block
      const unsigned char* br = s_r1 + (cb * 16 + c16) * TR_KQS + kk * 32;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 bhi = *reinterpret_cast<const bf16x8*>(br + s * 128);
        const bf16x8 blo = *reinterpret_cast<const bf16x8*>(br + s * 128 + 16);
        acc = mfma_bf16x3(ahi[s], alo[s], bhi, blo, acc);
      }
      const int tc = cb * 16 + c16;
      const int slot = s_dep[tc] - 1;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if ((rm[r] >> tc) & 1ull) dst[ro[r] + slot] = acc[r];
    }
  }
  if (RP && pn > 0) {
#pragma unroll
    for (int h = 0; h < NH; ++h) replay(h);
  }
  __syncthreads();  // (B_c) packed Gram rows, V rows

  // ---------- packed Ti and M2 rows on one or two waves; the others: S0 [K;Q]^T --
  // Trees deeper than 24 (one whole wave).  Lane c owns column c of Ti and M2.
  // Rows go in topological order from Ti = I - A Ti: row t is
  // e_t - sum_{k in anc(t)} A[t][k] Ti[k], A[t][k] = b_t Gamma(t,k) kk(t,k),
  // and row t of M2 is sum_{k in path(t)} Gamma(t,k) qk(t,k) Ti[k] with
  // Gamma(t,t) = 1.  Column c is nonzero only for c on t's path, at slot
  // dep(c) - 1, so lane c reads back only entries it wrote itself.  Per row,
  // lane 63 - j first finds the ancestor p_j at slot j (the j-th set bit of
  // t's ancestor mask), Gamma(t, p_j) by a DPP prefix product over the lanes
  // (deeper slots sit on lower lanes) and both coefficients; the row's sum
  // then takes them by readlane, with the Ti[p_j][c] reads going out eight at
  // a time.
  auto rlf = [](float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
  };
  auto solve_cols = [&](int h) {
    const float* s_gah = s_ga + h * TR_T;
    const float* s_gbh = s_gb + h * TR_T;
    const int c = lane;
    const bool live = c < T;
    const int dc = live ? s_dep[c] : 0;
    const int dm1 = live ? dc - 1 : TR_T;  // lowest ancestor slot that reaches column c
    const int jl = kWave - 1 - lane;       // the slot this lane prepares
    for (int t = 0; t < T; ++t) {
      const unsigned long long anc = s_anc[t];  // same address on every lane
      const int dt = s_dep[t], offt = s_off[t];
      const float at = s_gah[t], bt = s_gbh[t];
      const bool cpath = live && (c == t || ((anc >> c) & 1ull));
      // p_j, the j-th lowest set bit of anc, for j = jl < dt - 1
      const bool onj = jl < dt - 1;
      int r = onj ? jl : 0, pos = 0;
      unsigned w = static_cast<unsigned>(anc);
      {
        const int lo = __builtin_popcount(w);
        if (r >= lo) {
          r -= lo;
          pos = 32;
          w = static_cast<unsigned>(anc >> 32);
        }
      }
#pragma unroll
      for (int sh = 16; sh >= 1; sh >>= 1) {
        const int n = __builtin_popcount(w & ((1u << sh) - 1u));
        if (r >= n) {
          r -= n;
          pos += sh;
          w >>= sh;
        }
      }
      const int pj = onj ? pos : 0;
      const float aj = onj ? s_gah[pj] : 1.f;
      const int offj = s_off[pj];
      const float kkj = s_KK[offt + (onj ? jl : 0)];
      const float qkj = s_QK[offt + (jl < dt ? jl : 0)];
      // inclusive prefix product over lanes 0..lane (slots jl..63), then
      // shifted one lane: Gamma(t, p_j) / a_t = prod_{j < m < dt-1} a(p_m)
      float xs = aj;
      xs *= dpp_move<0x111, 0xF>(xs);  // row_shr:1
      xs *= dpp_move<0x112, 0xF>(xs);  // row_shr:2
      xs *= dpp_move<0x114, 0xF>(xs);  // row_shr:4
      xs *= dpp_move<0x118, 0xF>(xs);  // row_shr:8
      xs *= dpp_move<0x142, 0xA>(xs);  // row_bcast:15 into rows 1 and 3
      xs *= dpp_move<0x143, 0xC>(xs);  // row_bcast:31 into rows 2 and 3
      const float gj = at * dpp_move<0x138, 0xF>(xs);  // wave_shr:1
      const float cA = gj * kkj, cM = gj * qkj;
      float acc = 0.f, mac = 0.f;
      for (int j0 = 0; j0 < dt - 1; j0 += 8) {
        float xk[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = j0 + u < dt - 1 ? j0 + u : dt - 2;
          const int ok = __builtin_amdgcn_readlane(offj, kWave - 1 - j);
          xk[u] = s_TI[j >= dm1 ? ok + dc - 1 : 0];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = j0 + u < dt - 1 ? j0 + u : dt - 2;
          const float x = (j0 + u < dt - 1 && j >= dm1) ? xk[u] : 0.f;
          acc = fmaf(rlf(cA, kWave - 1 - j), x, acc);
          mac = fmaf(rlf(cM, kWave - 1 - j), x, mac);
        }
      }
      const float xt = (c == t ? 1.f : 0.f) - bt * acc;
      if (cpath) {
        s_TI[offt + dc - 1] = xt;
        s_M2[offt + dc - 1] = fmaf(rlf(qkj, kWave - dt), xt, mac);
      }
    }
  };
  // Depths 9 to 24 (17 to 24 in the replay forms, which solve 9 to 16 in
  // registers below): lane t solves its own row along its path, backward for
  // Ti and forward for M2, walking the path from the ancestor mask.  The
  // rows run side by side, so the cost grows with the square of the deepest
  // path; deeper trees take the column form above, whose cost follows the
  // summed path lengths (on 64-node trees with one long chain the two meet
  // near depth 24; a 64-node chain runs 3.1x faster in the column form).
  auto solve_path = [&](int h) {
    const float* s_gah = s_ga + h * TR_T;
    const float* s_gbh = s_gb + h * TR_T;
    const int t = lane;
    if (t >= T) return;
    const int d = s_dep[t];
    const int off = s_off[t];
    const unsigned long long mask = s_anc[t] | (1ull << t);
    s_TI[off + d - 1] = 1.f;
    for (int i = d - 2; i >= 0; --i) {
      unsigned long long mm = mask;
      for (int c = 0; c <= i; ++c) mm &= mm - 1ull;  // drop p_0 .. p_i
      float acc = 0.f, gmm = 1.f;
      for (int j = i + 1; j < d; ++j) {
        const int v = __builtin_ctzll(mm);
        mm &= mm - 1ull;
        gmm *= s_gah[v];
        acc = fmaf(s_TI[off + j] * s_gbh[v] * gmm, s_KK[s_off[v] + i], acc);
      }
      s_TI[off + i] = -acc;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int i = 0; i < d; ++i) {
      unsigned long long mm = mask;
      float acc = 0.f, gmm = 1.f;
      for (int j = d - 1; j >= i; --j) {
        const int v = 63 - __builtin_clzll(mm);
        mm ^= 1ull << v;
        acc = fmaf(gmm * s_QK[off + j], s_TI[s_off[v] + i], acc);
        gmm *= s_gah[v];
      }
      s_M2[off + i] = acc;
    }
  };
  // Depths 9 to 16 in the replay forms (one whole wave): lane t solves its
  // own row with the path's offsets and gates in registers; each row step's
  // Gram entries are read from LDS together.  The Ti rows go out first, and
  // M2 then reads the ancestors' Ti rows back from LDS (a wave's LDS accesses
  // run in order).  The plain two-head form would spill with it.
  auto solve_rows16 = [&](int h) {
    const float* s_gah = s_ga + h * TR_T;
    const float* s_gbh = s_gb + h * TR_T;
    const int t = lane;
    const int d = t < T ? s_dep[t] : 0;
    const int off = s_off[t];
    int po[16];
    float pa[16], pb[16];
    {
      unsigned long long mm = t < T ? (s_anc[t] | (1ull << t)) : 0ull;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int v = mm ? __builtin_ctzll(mm) : 0;
        mm &= mm - 1ull;
        pa[m] = s_gah[v];
        pb[m] = s_gbh[v];
        po[m] = m < d ? s_off[v] : 0;
      }
    }
    // Row t of Ti: x_{d-1} = 1, x_i = -sum_{j>i} x_j b_j Gamma(j,i) kk(j,i)
    float xs[16];
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      float kv[16];
#pragma unroll
      for (int j = i + 1; j < 16; ++j) kv[j] = s_KK[po[j] + i];
      float acc = 0.f, gmm = 1.f;
#pragma unroll
      for (int j = i + 1; j < 16; ++j) {
        gmm *= pa[j];
        acc = fmaf(xs[j] * pb[j] * gmm, j < d ? kv[j] : 0.f, acc);
      }
      xs[i] = (i == d - 1) ? 1.f : (i < d - 1 ? -acc : 0.f);
      __builtin_amdgcn_sched_barrier(0);  // one row step's reads at a time
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (t < T && i < d) s_TI[off + i] = xs[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // Row t of M2: sum_{j>=i} Gamma(t,p_j) qk(t,p_j) Ti[p_j][i]
    float oc[16];
    {
      float gmm = 1.f;
#pragma unroll
      for (int j = 15; j >= 0; --j) {
        oc[j] = (j < d) ? gmm * s_QK[off + j] : 0.f;
        if (j < d) gmm *= pa[j];
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int j = i; j < 16; ++j) acc = fmaf(oc[j], j < d ? s_TI[po[j] + i] : 0.f, acc);
      if (t < T && i < d) s_M2[off + i] = acc;
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto solve_rows = [&](int h) {
    if constexpr (RP) {
      if (s_maxd <= 16) {
        solve_rows16(h);
        return;
      }
    }
    if (s_maxd > 24)
      solve_cols(h);
    else
      solve_path(h);
  };
  // A head's rows for trees of depth <= 8, solved by one wave in registers
  // (ancestors' Ti rows come from their lanes by shuffle) and written to the
  // packed rows by store_rows_reg.
  auto solve_rows_reg = [&](int h, float* xs, float* m2) {
    const float* s_gah = s_ga + h * TR_T;
    const float* s_gbh = s_gb + h * TR_T;
    const int t = lane;
    const int d = t < T ? s_dep[t] : 0;
    const int off = s_off[t];
    const unsigned long long mask = t < T ? (s_anc[t] | (1ull << t)) : 0ull;
    int pn[8], po[8];
    float pa[8], pb[8];
    unsigned long long mm = mask;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int v = mm ? __builtin_ctzll(mm) : 0;
      mm &= mm - 1ull;
      pn[m] = v;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      pa[m] = s_gah[pn[m]];
      pb[m] = s_gbh[pn[m]];
      po[m] = s_off[pn[m]];
    }
    float kv[8][8];
#pragma unroll
    for (int j = 1; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < j; ++i) kv[j][i] = (j < d) ? s_KK[po[j] + i] : 0.f;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      float acc = 0.f, gmm = 1.f;
#pragma unroll
      for (int j = i + 1; j < 8; ++j) {
        gmm *= pa[j];
        acc = fmaf(xs[j] * pb[j] * gmm, kv[j][i], acc);
      }
      xs[i] = (i == d - 1) ? 1.f : (i < d - 1 ? -acc : 0.f);
    }
    float oc[8];
    {
      float gmm = 1.f;
#pragma unroll
      for (int j = 7; j >= 0; --j) {
        oc[j] = (j < d) ? gmm * s_QK[off + j] : 0.f;
        if (j < d) gmm *= pa[j];
      }
    }
    // Ti[p_j][i] is slot i of lane p_j's row (every lane takes part)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int j = i; j < 8; ++j) {
        const float tv = __shfl(xs[i], pn[j], 64);
        acc = fmaf(oc[j], (j < d) ? tv : 0.f, acc);
      }
      m2[i] = acc;
    }
  };
  auto store_rows_reg = [&](const float* xs, const float* m2) {
    const int t = lane;
    if (t < T) {
      const int d = s_dep[t], off = s_off[t];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < d) {
          s_TI[off + i] = xs[i];
          s_M2[off + i] = m2[i];
        }
    }
  };
  // Trees of depth <= 8 solve in registers on waves 2 (head 0, rows stored
  // at once) and 3 (head 1, rows stored once head 0's are expanded): the
  // waves that finish their share of the first products earliest, so the
  // solves leave the barrier's critical path.  Deeper trees solve on wave 0.
  float xs1[NH > 1 ? 8 : 1], m21[NH > 1 ? 8 : 1];
  const bool early = s_maxd <= 8;
  const bool early1 = NH > 1 && early;
  if (early) {
    if (wave == 2) {
      float xs0[8], m20[8];
      solve_rows_reg(0, xs0, m20);
      store_rows_reg(xs0, m20);
    }
    if constexpr (NH > 1) {
      if (wave == 3) solve_rows_reg(1, xs1, m21);
    }
  } else if (wave == 0) {
    solve_rows(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // S0 [K;Q]^T: A = this wave's tile of head h, B = pre-split k rows then q rows.
  auto s0_product = [&](int h, floatx4* acc) {
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 ahi, alo;
      split_bf16x8_pk(sreg[h][2 * s], sreg[h][2 * s + 1], ahi, alo);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const unsigned char* br = s_r1 + (cb * 16 + c16) * TR_KQS + kk * 32 + s * 128;
        const bf16x8 bhi = *reinterpret_cast<const bf16x8*>(br);
        const bf16x8 blo = *reinterpret_cast<const bf16x8*>(br + 16);
        acc[cb] = mfma_bf16x3(ahi, alo, bhi, blo, acc[cb]);
      }
    }
  };
  // RHS_t[i] = b_t (v_t[i] - gamma_t (S0 k_t)[i]) in place of v (own rows).
  auto form_rhs = [&](int h, const floatx4* acc) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int t = cb * 16 + c16;
      const float bt = s_gb[h * TR_T + t];
      const float gm = s_gam[h * TR_T + t];
      float* col = s_v + (wave * 16 + 4 * kk) * TR_VLD + (t ^ vsw(wave * 16 + 4 * kk));
#pragma unroll
      for (int r = 0; r < 4; ++r) col[r * TR_VLD] = bt * (col[r * TR_VLD] - gm * acc[cb][r]);
    }
  };
  // packed Ti and M2 rows expanded to a dense pre-split [Ti; M2] operand in
  // the K/Q space
  auto dense_operand = [&]() {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + q * TR_NT;  // (row n, step st, lane group kg)
      const int n = e / 8, st = (e / 4) % 2, kg = e % 4;
      const int nn = n % TR_T;
      const bool m2 = n >= TR_T;
      const unsigned long long mask = nn < T ? (s_anc[nn] | (1ull << nn)) : 0ull;
      const int off = s_off[nn];
      const float* src = m2 ? s_M2 : s_TI;
      float vv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int sidx = 32 * st + 8 * kg + i;
        const bool on = (mask >> sidx) & 1ull;
        const float val = src[on ? off + s_dep[sidx] - 1 : 0];
        vv[i] = on ? val : 0.f;
      }
      uint2 h0, l0, h1, l1;
      split4(vv, h0, l0);
      split4(vv + 4, h1, l1);
      unsigned char* dst = s_r1 + n * TR_B2S + (st * 4 + kg) * 32;
      *reinterpret_cast<uint4*>(dst) = make_uint4(h0.x, h0.y, h1.x, h1.y);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(l0.x, l0.y, l1.x, l1.y);
    }
  };
  // RHS^T [Ti; M2]^T on bf16x3 MFMA; u and o of head h from registers
  // (o adds gamma_t (S0 q_t) from the first product's q columns)
  auto second_product = [&](int h, const floatx4* acc1) {
    floatx4 acc2[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc2[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const float* ar = s_v + (wave * 16 + c16) * TR_VLD + ((32 * st + 8 * kk) ^ vsw(wave * 16 + c16));
      bf16x8 ahi, alo;
      split_bf16x8_pk(*reinterpret_cast<const floatx4*>(ar), *reinterpret_cast<const floatx4*>(ar + 4), ahi, alo);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const unsigned char* br = s_r1 + (cb * 16 + c16) * TR_B2S + (st * 4 + kk) * 32;
        const bf16x8 bhi = *reinterpret_cast<const bf16x8*>(br);
        const bf16x8 blo = *reinterpret_cast<const bf16x8*>(br + 16);
        acc2[cb] = mfma_bf16x3(ahi, alo, bhi, blo, acc2[cb]);
      }
    }
    const int i0 = wave * 16 + 4 * kk;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int t = (cb * 16 + c16) % TR_T;
      if (t < T) {
        const size_t oi = ((lb * T + t) * p.Hv + hv + h) * TR_D + i0;
        floatx4 val = acc2[cb];
        if (cb >= 4) val += s_gam[h * TR_T + t] * acc1[cb];
        // regular stores: the other 64 bytes of each 128-byte line come from
        // the neighbouring wave and are merged in L2 before the line is written
        *reinterpret_cast<floatx4*>((cb < 4 ? p.tu : p.o) + oi) = val;
      }
    }
  };

  floatx4 acc1[8];
  // the second head's product runs while K/Q are still in LDS, on the same
  // operand fragments as the first's; its RHS waits for the V space
  floatx4 acc1b[NH > 1 ? 8 : 1];
  if constexpr (NH > 1) {
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      acc1[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
      acc1b[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 ahi0, alo0, ahi1, alo1;
      split_bf16x8_pk(sreg[0][2 * s], sreg[0][2 * s + 1], ahi0, alo0);
      split_bf16x8_pk(sreg[1][2 * s], sreg[1][2 * s + 1], ahi1, alo1);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const unsigned char* br = s_r1 + (cb * 16 + c16) * TR_KQS + kk * 32 + s * 128;
        const bf16x8 bhi = *reinterpret_cast<const bf16x8*>(br);
        const bf16x8 blo = *reinterpret_cast<const bf16x8*>(br + 16);
        acc1[cb] = mfma_bf16x3(ahi0, alo0, bhi, blo, acc1[cb]);
        acc1b[cb] = mfma_bf16x3(ahi1, alo1, bhi, blo, acc1b[cb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    s0_product(0, acc1);
  }
  form_rhs(0, acc1);
  // The rolled tiles go back to the live state where the stores cost least:
  // the other waves while they wait for the solving waves at the barrier
  // below, the solving waves (2 and 3, or 0 for deep trees) once past it
  // (their stores then drain under the dense operand).
  const bool solver = early ? (wave == 2 || (NH > 1 && wave == 3)) : wave == 0;
  if (RP && pn > 0 && !solver) store_replayed();
  __syncthreads();  // (B_d) packed Ti, M2; RHS; K/Q space free
  if (RP && pn > 0 && solver) store_replayed();

  dense_operand();
  __syncthreads();  // (B_e)
  if constexpr (NH > 1) {
    // the second head's packed rows (the first head's are expanded)
    if (early1) {
      if (wave == 3) store_rows_reg(xs1, m21);
    } else if (wave == 0) {
      solve_rows(1);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  second_product(0, acc1);
  if constexpr (NH > 1) {
    __syncthreads();  // (B_f) head 0 done with V / RHS and [Ti; M2]; head 1 rows solved
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int t = (gr + 32 * (4 + r)) % TR_T;
#pragma unroll
      for (int e = 0; e < 8; ++e) s_v[(8 * li + e) * TR_VLD + (t ^ vsw(8 * li))] = vout[2 + r][e];
    }
    __syncthreads();  // (B_g) head 1's V rows
    form_rhs(1, acc1b);
    dense_operand();
    __syncthreads();  // (B_h)
    second_product(1, acc1b);
  }
}

// Without the replay, one workgroup per CU (the LDS allows no more) walks
// the units bid = blockIdx.x, blockIdx.x + gridDim.x, ...: the next unit's
// loads start right after the barrier instead of after a new workgroup's
// dispatch.  The grid is a multiple of the XCD count, so a workgroup's units
// all map to its own XCD.  The replay forms run one unit per workgroup: they
// sit at the register limit, and the loop made them spill.
template <int KC, bool RP, int NH, bool VG>
__global__ __launch_bounds__(TR_NT) void k_verify_tree(VerifyArgs p, int nbid) {
  if constexpr (RP) {
    tree_unit<KC, RP, NH, VG>(p, blockIdx.x);
  } else {
    for (int bid = blockIdx.x; bid < nbid; bid += gridDim.x) {
      tree_unit<KC, RP, NH, VG>(p, bid);
      __syncthreads();  // every wave is done with this unit's LDS
    }
  }
}

// Workgroups of a persistent tree launch: one per CU of the current device.
int tree_grid(long long nbid) {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return static_cast<int>(nbid);
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      return static_cast<int>(nbid);
    cus[dev] = (n + kNumXcd - 1) / kNumXcd * kNumXcd;
  }
  return static_cast<int>(nbid < cus[dev] ? nbid : cus[dev]);
}

}  // namespace

hipError_t launch_verify_tree(const VerifyArgs& a, hipStream_t s) {
  const int G = a.Hv / a.Hk;
  const int n_units = a.L * a.B * a.Hk;
  // both v-heads of a k-head in one workgroup (q/k conv, norms and Gram done
  // once) where the layout fits: two v-heads per k-head, conv width 4
  const int nh = (G == 2 && a.K == 4) ? 2 : 1;
  const long long grid =
      static_cast<long long>((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * (G / nh);
  if (grid > 0x7fffffffLL || a.T > TR_T || a.T < 1) return hipErrorInvalidValue;
  const bool rp = a.prev_n_keep != nullptr;
  if (rp && (a.pT < 1 || a.pT > TR_T || !a.ptu || !a.ptk || !a.ptg || !a.S_out))
    return hipErrorInvalidValue;
  const int nbid = static_cast<int>(grid);
  const dim3 gd(rp ? nbid : tree_grid(grid)), bd(TR_NT);
  if (nh == 2) {
    if (rp) hipLaunchKernelGGL((k_verify_tree<4, true, 2, false>), gd, bd, 0, s, a, nbid);
    else hipLaunchKernelGGL((k_verify_tree<4, false, 2, false>), gd, bd, 0, s, a, nbid);
  } else if (a.K == 4) {
    if (rp) hipLaunchKernelGGL((k_verify_tree<4, true, 1, false>), gd, bd, 0, s, a, nbid);
    else hipLaunchKernelGGL((k_verify_tree<4, false, 1, false>), gd, bd, 0, s, a, nbid);
  } else {
    if (rp) hipLaunchKernelGGL((k_verify_tree<0, true, 1, false>), gd, bd, 0, s, a, nbid);
    else hipLaunchKernelGGL((k_verify_tree<0, false, 1, false>), gd, bd, 0, s, a, nbid);
  }
  return hipGetLastError();
}

hipError_t launch_verify_tree_vg(const VerifyArgs& a, hipStream_t s) {
  const int G = a.Hv / a.Hk;
  const int n_units = a.L * a.B * a.Hk;
  const long long grid = static_cast<long long>((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * G;
  if (grid > 0x7fffffffLL || a.T > TR_T || a.T < 1) return hipErrorInvalidValue;
  const bool rp = a.prev_n_keep != nullptr;
  if (rp && (a.pT < 1 || a.pT > TR_T || !a.ptu || !a.ptk || !a.ptg || !a.S_out))
    return hipErrorInvalidValue;
  const int nbid = static_cast<int>(grid);
  const dim3 gd(rp ? nbid : tree_grid(grid)), bd(TR_NT);
  if (a.K == 4) {
    if (rp) hipLaunchKernelGGL((k_verify_tree<4, true, 1, true>), gd, bd, 0, s, a, nbid);
    else hipLaunchKernelGGL((k_verify_tree<4, false, 1, true>), gd, bd, 0, s, a, nbid);
  } else {
    if (rp) hipLaunchKernelGGL((k_verify_tree<0, true, 1, true>), gd, bd, 0, s, a, nbid);
    else hipLaunchKernelGGL((k_verify_tree<0, false, 1, true>), gd, bd, 0, s, a, nbid);
  }
  return hipGetLastError();
}

}  // namespace gdn
