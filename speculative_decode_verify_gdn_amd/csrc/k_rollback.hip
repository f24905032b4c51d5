// k_rollback.hip -- tape-replay rollback of the gated delta state and of the
// conv window, for gfx950 (GDN page s4, "Tape-Replay rollback").
//
// State: the live buffer still holds the pre-verify snapshot S0.  Replaying
// the accepted steps p_0..p_{n-1} from the tape,
//   S <- g_{p_i} S + u_{p_i} k_{p_i}^T,
// unrolls to one closed form,
//   S_n = w_{-1} S0 + sum_i w_i u_{p_i} k_{p_i}^T,   w_i = prod_{j>i} g_{p_j},
// so each element costs one read of S0, n fused multiply-adds against the
// tape, and one write -- no products with the state.  n = 0 returns before
// touching the state, so the cost is one state pass plus O(n) tape bytes.
//
// Layout: one 256-thread workgroup per (layer, seq, v-head, RB-row block)
// -- for tapes of at most 16 steps, per (several layers, seq, v-head, row
// block), walked in turn, so that a sequence that accepted nothing costs
// few workgroups; every thread owns 4 float4 of the block, read and written
// fully coalesced (whole cache lines), and many small workgroups per CU keep
// the state streaming.  The block's n tape rows (k: n x Dk, w-scaled u: n x RB) are
// staged in LDS, the rank-n update U = sum_i w_i u_i k_i^T is formed on fp32
// MFMA (four steps per instruction), and it reaches the threads' layout
// through LDS: S_n = gamma S0 + U.
//
// Conv window: new row j = row n+j of [old window; x[p_0]; ...; x[p_{n-1}]],
// copied 16 bytes per thread by one workgroup per (several layers, seq);
// all sources are loaded before any store, so the in-place update is safe.

#include "gdn_common.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

// LT (tapes longer than 16 steps, several staging chunks): each chunk's
// loads all go out together, at a lower occupancy; shorter tapes keep one
// load per thread in flight and eight waves per SIMD.
template <int DK, int DV, bool LT>
__device__ __forceinline__ void tape_rollback_body(const RollbackArgs& p, int bid) {
  constexpr int NT = 256;
  constexpr int VPT = 4;                  // float4 per thread
  constexpr int RB0 = NT * VPT * 4 / DK;  // rows that fill the block
  constexpr int RB = RB0 < DV ? RB0 : DV;
  constexpr int NRBLK = DV / RB;
  constexpr int C4 = DK / 4;              // float4 per row
  constexpr int NV = RB * C4;             // float4 in the block
  constexpr int CH = 16;                  // tape entries staged per chunk
  constexpr int TM = 64;                  // longest tape
  static_assert(DV % RB == 0 && NV <= NT * VPT, "row blocks");

  // the rank-n update on fp32 MFMA: 16x16 tiles of the RB x DK block, TPW
  // per wave; the tiles go to the thread layout of the state through LDS
  constexpr int NRT = RB / 16, NCT = DK / 16, TPW = NRT * NCT / 4;
  constexpr int ULD = DK + 4;  // padded row stride of the update in LDS
  constexpr int NSTAGE = CH * DK + CH * RB;
  constexpr int NBUF = NSTAGE > RB * ULD ? NSTAGE : RB * ULD;
  static_assert(NRT * NCT % 4 == 0, "tiles per wave");
  // staged tape (k rows, w-scaled u slice); reused for the update once the
  // products are done
  __shared__ __align__(16) float s_buf[NBUF];
  float* const s_k = s_buf;
  float* const s_u = s_buf + CH * DK;
  __shared__ float s_w[TM];
  __shared__ int s_pi[TM];
  __shared__ int s_bad;
  __shared__ float s_gam;
  static_assert(TM == kWave, "one lane per tape step");

  const int tid = threadIdx.x;
  int rblk, hv, bb, l0, l1;
  if constexpr (LT) {
    // long tapes: the G v-heads x NRBLK row blocks of one (layer, seq,
    // k-head) read the same k rows n times over; they take consecutive slots
    // of one XCD (workgroup i runs on XCD i mod 8) so the rows come from
    // that XCD's L2 after the first read
    const int G = p.Hv / p.Hk;
    const UnitSub us = xcd_unit_sub(bid, G * NRBLK);
    if (us.unit >= p.L * p.B * p.Hk) return;
    rblk = us.sub % NRBLK;
    hv = (us.unit % p.Hk) * G + us.sub / NRBLK;
    const int lb0 = us.unit / p.Hk;
    bb = lb0 % p.B;
    l0 = lb0 / p.B;
    l1 = l0 + 1;
  } else {
    // short tapes: layers l0 .. l0 + lpw - 1 of one (seq, v-head, row
    // block), in turn.  The accepted length is read once, so a sequence
    // that accepted nothing costs one workgroup per lpw layers.
    const int lpw = p.lpw > 0 ? p.lpw : 1;
    rblk = bid % NRBLK;
    int rest = bid / NRBLK;
    hv = rest % p.Hv;
    rest /= p.Hv;
    bb = rest % p.B;
    l0 = (rest / p.B) * lpw;
    l1 = l0 + lpw < p.L ? l0 + lpw : p.L;
  }
  const int T = p.T;
  const int n = p.n_keep ? p.n_keep[bb] : p.n_all;
  const bool reporter = l0 == 0 && hv == 0 && rblk == 0;
  if (n == 0) return;
  if (n < 0 || n > T) {
    if (tid == 0 && p.dev_err && reporter) atomicOr(p.dev_err, GDN_DEV_ERR_N_KEEP);
    return;
  }
  const int hk = hv / (p.Hv / p.Hk);
  const int r0 = rblk * RB;
  float* Sblk = nullptr;

  // Snapshot loads first (unconditional: every thread owns VPT float4).
  floatx4 sv[VPT];
  auto load_sv = [&](size_t lb, int t) {
    Sblk = p.S + ((lb * p.Hv + hv) * DV + r0) * static_cast<size_t>(DK);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const int e = t + v * NT;
      sv[v] = reinterpret_cast<const floatx4*>(Sblk)[e < NV ? e : 0];
    }
  };
  load_sv(static_cast<size_t>(l0) * p.B + bb, tid);

  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (tid < n) {
    const int pi = p.path ? p.path[static_cast<size_t>(bb) * T + tid] : tid;
    if (pi < 0 || pi >= T) s_bad = 1;
    s_pi[tid] = pi < 0 ? 0 : (pi >= T ? T - 1 : pi);
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0 && p.dev_err && reporter) atomicOr(p.dev_err, GDN_DEV_ERR_PATH);
    return;
  }
  for (int l = l0; l < l1; ++l) {
  const size_t lb = static_cast<size_t>(l) * p.B + bb;
  // short tapes: an opaque copy of the lane index per layer, so that
  // lane-dependent addresses are formed inside the loop rather than held
  // across it (long tapes run one layer)
  int tid = threadIdx.x;
  if constexpr (!LT) asm volatile("" : "+v"(tid));
  if (l > l0) load_sv(lb, tid);
  if (tid < kWave) {
    // wave 0, one lane per step: every gate load in flight at once, then
    // w_i = prod_{j>i} g_{p_j} by a suffix-product scan (shuffles on every
    // lane) and gamma = prod_j g_{p_j}
    const float gv = tid < n ? p.tg[(lb * T + s_pi[tid]) * p.Hv + hv] : 1.f;
    float xs = gv;  // inclusive suffix product prod_{j >= lane} g_j
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const float y = __shfl_down(xs, o, kWave);
      if (tid + o < kWave) xs *= y;
    }
    float w = __shfl_down(xs, 1, kWave);
    if (tid == kWave - 1) w = 1.f;
    if (tid < n) s_w[tid] = w;
    if (tid == 0) s_gam = xs;
  }
  __syncthreads();
  const float gam = s_gam;
  const int wave = tid / kWave, lane = tid % kWave;
  const int c16 = lane & 15, kk = lane >> 4;
  // U = sum_i (w_i u_i) k_i^T as transposed tiles D[j][r] = sum_i k_i[j]
  // (w_i u_i)[r] on mfma_f32_16x16x4f32 (four steps per instruction): lane
  // (c16, kk) of tile (rt, ct) ends holding U[16 rt + c16][16 ct + 4 kk .. +3]
  floatx4 ut[TPW];
#pragma unroll
  for (int m = 0; m < TPW; ++m) ut[m] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int i0 = 0; i0 < n; i0 += CH) {
    const int nc = n - i0 < CH ? n - i0 : CH;
    if (i0 > 0) __syncthreads();  // previous chunk consumed
    if constexpr (LT) {
      // every load of the chunk first (clamped, valid addresses), then the
      // LDS stores
      constexpr int KPT = (CH * C4 + NT - 1) / NT;  // k float4 per thread
      constexpr int UPT = (CH * RB + NT - 1) / NT;  // u floats per thread
      floatx4 kr[KPT];
      float ur[UPT];
#pragma unroll
      for (int q = 0; q < KPT; ++q) {
        const int e = tid + q * NT;
        const int i = e < nc * C4 ? e / C4 : nc - 1, c4 = e % C4;
        kr[q] = reinterpret_cast<const floatx4*>(p.tk + ((lb * T + s_pi[i0 + i]) * p.Hk + hk) * DK)[c4];
      }
#pragma unroll
      for (int q = 0; q < UPT; ++q) {
        const int e = tid + q * NT;
        const int i = e < nc * RB ? e / RB : nc - 1, r = e % RB;
        ur[q] = s_w[i0 + i] * p.tu[((lb * T + s_pi[i0 + i]) * p.Hv + hv) * DV + r0 + r];
      }
#pragma unroll
      for (int q = 0; q < KPT; ++q) {
        const int e = tid + q * NT;
        if (e < nc * C4) reinterpret_cast<floatx4*>(s_k)[e] = kr[q];
      }
#pragma unroll
      for (int q = 0; q < UPT; ++q) {
        const int e = tid + q * NT;
        if (e < nc * RB) s_u[e] = ur[q];
      }
    } else {
      for (int e = tid; e < nc * C4; e += NT) {
        const int i = e / C4, c4 = e % C4;
        reinterpret_cast<floatx4*>(s_k)[e] =
            reinterpret_cast<const floatx4*>(p.tk + ((lb * T + s_pi[i0 + i]) * p.Hk + hk) * DK)[c4];
      }
      for (int e = tid; e < nc * RB; e += NT) {
        const int i = e / RB, r = e % RB;
        s_u[e] = s_w[i0 + i] * p.tu[((lb * T + s_pi[i0 + i]) * p.Hv + hv) * DV + r0 + r];
      }
    }
    __syncthreads();
    for (int s4 = 0; s4 < nc; s4 += 4) {
      const int i = s4 + kk;  // this lane's step; steps past the chunk add zero
      const bool on = i < nc;
      const int ii = on ? i : 0;
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        const int j = wave * TPW + m;
        const int rt = j / NCT, ct = j % NCT;
        const float a = s_k[ii * DK + 16 * ct + c16];
        const float b = s_u[ii * RB + 16 * rt + c16];
        ut[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(on ? a : 0.f, on ? b : 0.f, ut[m], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // every wave is done with the staged tape
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int j = wave * TPW + m;
    const int rt = j / NCT, ct = j % NCT;
    *reinterpret_cast<floatx4*>(s_buf + (16 * rt + c16) * ULD + 16 * ct + 4 * kk) = ut[m];
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int e = tid + v * NT;
    const int r = (e % NV) / C4, c = (e % C4) * 4;
    const floatx4 acc = sv[v] * gam + *reinterpret_cast<const floatx4*>(s_buf + r * ULD + c);
    if (e < NV) reinterpret_cast<floatx4*>(Sblk)[e] = acc;
  }
  }  // layers
}

// Short tapes: layers per workgroup.  As few workgroups as keep the chip
// streaming when every sequence replays (about 16K), since each launched
// workgroup costs its dispatch and one load even when its sequence accepted
// nothing.
template <int DK, int DV>
int rb_layers(const RollbackArgs& a) {
  constexpr int RB0 = 256 * 4 * 4 / DK;
  constexpr int NRBLK = DV / (RB0 < DV ? RB0 : DV);
  const long long units = static_cast<long long>(a.L) * a.B * a.Hv * NRBLK;
  const long long lpw = (units + 16383) / 16384;
  return static_cast<int>(lpw < 1 ? 1 : (lpw > a.L ? a.L : lpw));
}

// Workgroups of the state rollback: short tapes, one per (lpw layers, seq,
// v-head, row block); long tapes, one per (layer, seq, v-head, row block),
// the (layer, seq, k-head) units rounded up to a multiple of the XCD count.
// The returned args carry the layers per workgroup.
template <int DK, int DV>
long long state_grid(const RollbackArgs& a, RollbackArgs* out = nullptr) {
  constexpr int RB0 = 256 * 4 * 4 / DK;
  constexpr int NRBLK = DV / (RB0 < DV ? RB0 : DV);
  if (out) *out = a;
  if (a.T > 16) {
    const long long units = static_cast<long long>(a.L) * a.B * a.Hk;
    const long long padded = (units + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (out) out->lpw = 1;
    return padded * (a.Hv / a.Hk) * NRBLK;
  }
  const int lpw = rb_layers<DK, DV>(a);
  if (out) out->lpw = lpw;
  return static_cast<long long>((a.L + lpw - 1) / lpw) * a.B * a.Hv * NRBLK;
}

template <int DK, int DV, bool LT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LT ? 7 : 8))) void k_tape_rollback(RollbackArgs p) {
  tape_rollback_body<DK, DV, LT>(p, blockIdx.x);
}

template <int DK, int DV>
hipError_t launch_rb(const RollbackArgs& a0, hipStream_t s) {
  RollbackArgs a;
  const long long grid = state_grid<DK, DV>(a0, &a);
  if (grid > 0x7fffffffLL || a.T > 64) return hipErrorInvalidValue;
  if (a.T > 16) hipLaunchKernelGGL((k_tape_rollback<DK, DV, true>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_tape_rollback<DK, DV, false>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Per-key-channel decay (the [B,T,Hv,Dk] decay tape): the closed form
// becomes S_n = S0 diag(gamma) + sum_i u_{p_i} (k_{p_i} o w_i)^T with
// w_i[c] = prod_{j>i} g_{p_j}[c] and gamma[c] = prod_j g_{p_j}[c].  One
// thread per key channel forms the weights backwards along the path and
// stages k o w for all n <= 64 steps at once; the state pass is as above.
template <int DK, int DV, int TM>
__global__ __launch_bounds__(256) void k_tape_rollback_vg(RollbackArgs p) {
  constexpr int NT = 256;
  constexpr int VPT = 4;
  constexpr int RB0 = NT * VPT * 4 / DK;
  constexpr int RB = RB0 < DV ? RB0 : DV;
  constexpr int NRBLK = DV / RB;
  constexpr int C4 = DK / 4;
  constexpr int NV = RB * C4;
  // TM: longest tape staged (16 for rounds of up to 16 drafts, else 64); the
  // k * w staging is sized to it so that short tapes keep more workgroups
  // resident
  static_assert(DV % RB == 0 && NV <= NT * VPT && DK <= NT, "row blocks");

  __shared__ __align__(16) float s_kw[TM * DK];
  __shared__ float s_u[TM * RB];
  __shared__ __align__(16) float s_gam[DK];
  __shared__ int s_pi[TM];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int rblk = blockIdx.x % NRBLK;
  const int rest = blockIdx.x / NRBLK;
  const int hv = rest % p.Hv;
  const size_t lb = rest / p.Hv;
  const int bb = static_cast<int>(lb % p.B);
  const int l = static_cast<int>(lb / p.B);
  const int T = p.T;
  const int n = p.n_keep ? p.n_keep[bb] : p.n_all;
  if (n == 0) return;
  if (n < 0 || n > T) {
    if (tid == 0 && p.dev_err && l == 0 && hv == 0 && rblk == 0) atomicOr(p.dev_err, GDN_DEV_ERR_N_KEEP);
    return;
  }
  const int hk = hv / (p.Hv / p.Hk);
  const int r0 = rblk * RB;
  float* Sblk = p.S + ((lb * p.Hv + hv) * DV + r0) * static_cast<size_t>(DK);

  floatx4 sv[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int e = tid + v * NT;
    sv[v] = reinterpret_cast<const floatx4*>(Sblk)[e < NV ? e : 0];
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (tid < n) {
    const int pi = p.path ? p.path[static_cast<size_t>(bb) * T + tid] : tid;
    if (pi < 0 || pi >= T) s_bad = 1;
    s_pi[tid] = pi < 0 ? 0 : (pi >= T ? T - 1 : pi);
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0 && p.dev_err && l == 0 && hv == 0 && rblk == 0) atomicOr(p.dev_err, GDN_DEV_ERR_PATH);
    return;
  }
  if (tid < DK) {  // channel tid: weights backwards along the path
    float w = 1.f;
    for (int i1 = n; i1 > 0; i1 -= 16) {  // 16 steps' loads in flight at once
      const int i0 = i1 - 16 > 0 ? i1 - 16 : 0;
      float kv[16], gv[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = i1 - 1 - q;
        const size_t t = lb * T + s_pi[i >= i0 ? i : i0];
        kv[q] = p.tk[(t * p.Hk + hk) * DK + tid];
        gv[q] = p.tg[(t * p.Hv + hv) * DK + tid];
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = i1 - 1 - q;
        if (i >= i0) {
          s_kw[i * DK + tid] = kv[q] * w;
          w *= gv[q];
        }
      }
    }
    s_gam[tid] = w;
  }
  for (int e = tid; e < n * RB; e += NT) {
    const int i = e / RB, rr = e % RB;
    s_u[e] = p.tu[((lb * T + s_pi[i]) * p.Hv + hv) * DV + r0 + rr];
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int e = tid + v * NT;
    const int rr = (e % NV) / C4, c = (e % C4) * 4;
    floatx4 acc = sv[v] * *reinterpret_cast<const floatx4*>(s_gam + c);
    for (int i = 0; i < n; ++i) {
      const float u = s_u[i * RB + rr];
      const floatx4 k = *reinterpret_cast<const floatx4*>(s_kw + i * DK + c);
      acc[0] = fmaf(u, k[0], acc[0]);
      acc[1] = fmaf(u, k[1], acc[1]);
      acc[2] = fmaf(u, k[2], acc[2]);
      acc[3] = fmaf(u, k[3], acc[3]);
    }
    if (e < NV) reinterpret_cast<floatx4*>(Sblk)[e] = acc;
  }
}

template <int DK, int DV>
hipError_t launch_rb_vg(const RollbackArgs& a, hipStream_t s) {
  constexpr int RB0 = 256 * 4 * 4 / DK;
  constexpr int RB = RB0 < DV ? RB0 : DV;
  const long long grid = static_cast<long long>(a.L) * a.B * a.Hv * (DV / RB);
  if (grid > 0x7fffffffLL || a.T > 64) return hipErrorInvalidValue;
  if (a.T <= 16)
    hipLaunchKernelGGL((k_tape_rollback_vg<DK, DV, 16>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_tape_rollback_vg<DK, DV, 64>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// One workgroup per (lpw layers, seq): the window indices depend on the
// sequence only, so they are formed once; then every layer's rows are copied
// 16 bytes of channels per thread, CB chunks' loads in flight together.
// KM1 = K-1 window rows.
template <int ESZ, int KM1>
__device__ __forceinline__ void conv_rollback_body(const ConvRollbackArgs& p, int bid, int lpw) {
  constexpr int EPC = 16 / ESZ;  // elements per chunk
  constexpr int CB = KM1 <= 4 ? 8 / KM1 : 1;  // at most 8 rows of loads in flight (64 VGPRs)
  const int tid = threadIdx.x;
  const int bb = bid % p.B;
  const int l0 = (bid / p.B) * lpw;
  const int l1 = l0 + lpw < p.L ? l0 + lpw : p.L;
  const int n = p.n_keep ? p.n_keep[bb] : p.n_all;
  const int T = p.T;
  const bool first_block = l0 == 0;
  if (n < 0 || n > T) {
    if (first_block && tid == 0 && p.dev_err) atomicOr(p.dev_err, GDN_DEV_ERR_N_KEEP);
    return;
  }
  int idx[KM1];
  bool bad = false;
#pragma unroll
  for (int j = 0; j < KM1; ++j) {
    int id = n + j - KM1;  // position in [old rows; accepted rows], minus KM1
    if (id >= 0 && p.path) {
      id = p.path[static_cast<size_t>(bb) * T + id];
      if (id < 0 || id >= T) {
        bad = true;
        id = 0;
      }
    }
    idx[j] = id;
  }
  if (bad) {
    if (first_block && tid == 0 && p.dev_err) atomicOr(p.dev_err, GDN_DEV_ERR_PATH);
    return;
  }
  if (p.win_idx && first_block && tid == 0) {
#pragma unroll
    for (int j = 0; j < KM1; ++j) p.win_idx[static_cast<size_t>(bb) * KM1 + j] = idx[j];
  }
  if (n == 0) return;  // window unchanged
  const int row_chunks = p.C / EPC;
  const u32x4* xs = static_cast<const u32x4*>(p.x);
  u32x4* cs = static_cast<u32x4*>(p.conv_state);
  for (int l = l0; l < l1; ++l) {
    const size_t lb = static_cast<size_t>(l) * p.B + bb;
    u32x4* crow = cs + lb * KM1 * row_chunks;
    // each new row's source row (a select of addresses, so every load is
    // unconditional)
    const u32x4* src[KM1];
#pragma unroll
    for (int j = 0; j < KM1; ++j) {
      const int id = idx[j];
      src[j] = id < 0 ? crow + (KM1 + id) * row_chunks
                      : xs + lb * (p.x_ld / EPC) + static_cast<size_t>(id) * row_chunks;
    }
    // whole batches of CB chunks: every source first, then the stores; a
    // chunk's new rows come from its own old rows, so the in-place update
    // is safe
    int c0 = 0;
    for (; c0 + CB * 256 <= row_chunks; c0 += CB * 256) {
      u32x4 v[CB * KM1];
#pragma unroll
      for (int q = 0; q < CB; ++q)
#pragma unroll
        for (int j = 0; j < KM1; ++j) v[q * KM1 + j] = src[j][c0 + q * 256 + tid];
#pragma unroll
      for (int q = 0; q < CB; ++q)
#pragma unroll
        for (int j = 0; j < KM1; ++j) crow[j * row_chunks + c0 + q * 256 + tid] = v[q * KM1 + j];
    }
    // the rest, one chunk per thread
    for (int ch = c0 + tid; ch < row_chunks; ch += 256) {
      u32x4 v[KM1];
#pragma unroll
      for (int j = 0; j < KM1; ++j) v[j] = src[j][ch];
#pragma unroll
      for (int j = 0; j < KM1; ++j) crow[j * row_chunks + ch] = v[j];
    }
  }
}

// Layers per conv workgroup: as few as leave about 2K workgroups, so that a
// round in which few sequences accepted anything launches few of them.
inline int conv_layers(const ConvRollbackArgs& a) {
  const long long lpw = (static_cast<long long>(a.L) * a.B + 2047) / 2048;
  return static_cast<int>(lpw < 1 ? 1 : (lpw > a.L ? a.L : lpw));
}

template <int ESZ, int KM1>
__global__ __launch_bounds__(256) void k_conv_rollback(ConvRollbackArgs p, int lpw) {
  conv_rollback_body<ESZ, KM1>(p, blockIdx.x, lpw);
}

template <int ESZ>
hipError_t launch_crb(const ConvRollbackArgs& a, hipStream_t s) {
  const int lpw = conv_layers(a);
  const dim3 grid(static_cast<unsigned>((a.L + lpw - 1) / lpw) * a.B);
  switch (a.K) {
    case 2: hipLaunchKernelGGL((k_conv_rollback<ESZ, 1>), grid, dim3(256), 0, s, a, lpw); break;
    case 3: hipLaunchKernelGGL((k_conv_rollback<ESZ, 2>), grid, dim3(256), 0, s, a, lpw); break;
    case 4: hipLaunchKernelGGL((k_conv_rollback<ESZ, 3>), grid, dim3(256), 0, s, a, lpw); break;
    case 5: hipLaunchKernelGGL((k_conv_rollback<ESZ, 4>), grid, dim3(256), 0, s, a, lpw); break;
    case 6: hipLaunchKernelGGL((k_conv_rollback<ESZ, 5>), grid, dim3(256), 0, s, a, lpw); break;
    case 7: hipLaunchKernelGGL((k_conv_rollback<ESZ, 6>), grid, dim3(256), 0, s, a, lpw); break;
    case 8: hipLaunchKernelGGL((k_conv_rollback<ESZ, 7>), grid, dim3(256), 0, s, a, lpw); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tape_rollback(const RollbackArgs& a, int dk, int dv, hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 32: return launch_rb<32, 32>(a, s);
    case 64: return launch_rb<64, 64>(a, s);
    case 128: return launch_rb<128, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

namespace {

// Both rollbacks of a round in one launch: the conv-window workgroups first
// (few, each walking its layers, so they overlap the state pass), then the
// state ones.  Built for the common conv width (K = 4); other widths take
// the two launches.
template <int DK, int DV, int ESZ, bool LT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LT ? 7 : 8))) void k_round_rollback(RollbackArgs r, ConvRollbackArgs c,
                                                        int n_conv, int conv_lpw) {
  const int bid = blockIdx.x;
  if (bid < n_conv) {
    conv_rollback_body<ESZ, 3>(c, bid, conv_lpw);
  } else {
    tape_rollback_body<DK, DV, LT>(r, bid - n_conv);
  }
}

template <int DK, int DV>
hipError_t launch_rr(const RollbackArgs& r0, const ConvRollbackArgs& c, int dtype, hipStream_t s) {
  RollbackArgs r;
  const long long n_state = state_grid<DK, DV>(r0, &r);
  const int conv_lpw = conv_layers(c);
  const long long n_conv = static_cast<long long>((c.L + conv_lpw - 1) / conv_lpw) * c.B;
  const long long grid = n_conv + n_state;
  if (grid > 0x7fffffffLL || r.T > 64 || c.K != 4) return hipErrorInvalidValue;
  const int nc = static_cast<int>(n_conv);
  if (r.T > 16) {
    if (dtype == 1) hipLaunchKernelGGL((k_round_rollback<DK, DV, 2, true>), dim3(grid), dim3(256), 0, s, r, c, nc, conv_lpw);
    else hipLaunchKernelGGL((k_round_rollback<DK, DV, 4, true>), dim3(grid), dim3(256), 0, s, r, c, nc, conv_lpw);
  } else {
    if (dtype == 1) hipLaunchKernelGGL((k_round_rollback<DK, DV, 2, false>), dim3(grid), dim3(256), 0, s, r, c, nc, conv_lpw);
    else hipLaunchKernelGGL((k_round_rollback<DK, DV, 4, false>), dim3(grid), dim3(256), 0, s, r, c, nc, conv_lpw);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tape_rollback_vg(const RollbackArgs& a, int dk, int dv, hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 32: return launch_rb_vg<32, 32>(a, s);
    case 64: return launch_rb_vg<64, 64>(a, s);
    case 128: return launch_rb_vg<128, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_round_rollback(const RollbackArgs& r, const ConvRollbackArgs& c, int dk, int dv,
                                 int dtype, hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 32: return launch_rr<32, 32>(r, c, dtype, s);
    case 64: return launch_rr<64, 64>(r, c, dtype, s);
    case 128: return launch_rr<128, 128>(r, c, dtype, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv_rollback(const ConvRollbackArgs& a, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_crb<2>(a, s) : launch_crb<4>(a, s);
}

}  // namespace gdn
