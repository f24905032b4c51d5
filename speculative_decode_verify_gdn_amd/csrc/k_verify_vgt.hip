// k_verify_vgt.hip -- verify of a draft tree (or chain) of T <= 64 nodes
// through GDN layers whose decay gate acts per key channel, for gfx950,
// optionally replaying the previous round's accepted path onto the state
// first.
//
// Node v with parent p steps from p's state (GDN page s2.1, with the tape's
// per-key-channel gate form of s4):
//   S_v = S_p diag(a_v) + u_v k_v^T,  u_v = b_v (v_v - S_p diag(a_v) k_v),
//   o_v = S_v q_v,  S_{-1} = S0.
// Unrolled from the snapshot along v's root path: for an ancestor i of v let
// w_{v,i} be the elementwise product of a_j over the path nodes j below i, down
// to and including v, and gamma_v the product over the whole path.  Then
//   S_p diag(a_v) k_v = S0 (gamma_v * k_v) + sum_i u_i c_{v,i},
//   S_v q_v           = S0 (gamma_v * q_v) + sum_i u_i d_{v,i} + u_v (k_v . q_v),
// with the scalars c_{v,i} = sum_c k_i[c] w_{v,i}[c] k_v[c] and d_{v,i} the same
// with q_v.  Only forward products of gates appear -- no ratios -- so gates
// near zero cannot overflow it, and the state is never updated: each node
// costs two dot products of every state row with per-node vectors plus one
// multiply-add per ancestor, and S0 is read once.
//
// One workgroup per (layer, seq, v-head); 512 threads for 128-dim heads, 256
// otherwise.  Thread (row r, part h) holds a slice of S0 row r in registers:
// float4 column groups 4h + 4*TPR*m, so the parts of a row read adjacent LDS
// words.  Nodes go through in chunks of 16:
//   conv + SiLU of the chunk's q, k, v channels (window rows read from the
//     input, node then ancestors then old conv rows),
//   L2 norms, one wave per node (k goes to the tape),
//   path coefficients, one wave per node, walking up the ancestors,
//   the rows: each node in order; u of every node stays in LDS so that its
//     descendants can read it.
// With a previous accepted path (replay), its tape entries are staged in LDS
// and S <- S diag(g_i) + u_i k_i^T is applied in registers to the snapshot,
// which is written back in place before the verify reads it.

#include "gdn_common.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

constexpr int kVtT = 64;  // nodes per tree (max)
constexpr int kVtC = 16;  // nodes per chunk

template <int D>
constexpr int vgt_threads() {
  return D == 128 ? 512 : 256;
}

// Four consecutive input elements widened to fp32.
template <typename TIn>
struct Quad;
template <>
struct Quad<uint16_t> {
  static __device__ __forceinline__ floatx4 load(const uint16_t* p) {
    const uint2 r = *reinterpret_cast<const uint2*>(p);
    return floatx4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                   __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
  }
};
template <>
struct Quad<float> {
  static __device__ __forceinline__ floatx4 load(const float* p) {
    return *reinterpret_cast<const floatx4*>(p);
  }
};

// Sums over aligned groups of 2, 4, 8 or 16 lanes with DPP moves (VALU
// latency, unlike LDS-routed shuffles); every lane gets its group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if (N >= 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  if (N >= 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  if (N >= 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  if (N >= 16) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// Sum over the 64 lanes (uniform result): 16-lane sums, then the four rows.
__device__ __forceinline__ float wave_total(float v) {
  v = group_sum<16>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
}

__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int KC, typename TIn, bool RP>
__global__ __launch_bounds__(vgt_threads<D>()) void k_verify_vgt(VerifyArgs p) {
  constexpr int NT = vgt_threads<D>();
  constexpr int TPR = NT / D;  // threads per state row
  constexpr int CPT = D / TPR;  // columns per thread
  constexpr int NQ = CPT / 4;   // float4 column groups per thread
  constexpr int NWV = NT / kWave;
  constexpr int KM = KC > 0 ? KC : 8;
  constexpr int MPL = (D + kWave - 1) / kWave;  // channels per lane, wave-per-node phases
  constexpr int NG = 3 * D / 4;                 // 4-channel conv groups per node
  static_assert(CPT % 4 == 0 && NWV >= 2 && TPR <= 16, "layout");

  __shared__ __align__(16) float s_k[kVtT][D];   // normalised k of every node
  __shared__ __align__(16) float s_a[kVtT][D];   // gates of every node
  __shared__ __align__(16) float s_u[kVtT][D];   // u of every node, [node][row]
  __shared__ __align__(16) float s_q[kVtC][D];   // the chunk's normalised q
  __shared__ __align__(16) float s_v[kVtC][D];   // the chunk's v
  __shared__ __align__(16) float s_gk[kVtC][D];  // gamma_v * k_v
  __shared__ __align__(16) float s_gq[kVtC][D];  // gamma_v * q_v
  __shared__ float s_c[kVtC][kVtT], s_d[kVtC][kVtT];  // c_{v,i}, d_{v,i} by ancestor slot
  __shared__ int s_ai[kVtC][kVtT];                    // ancestor of each slot
  __shared__ __align__(16) float s_w[3 * D * KM];     // conv weights [channel][tap]
  __shared__ int s_par[kVtT], s_widx[kVtT * KM];
  __shared__ float s_b[kVtT], s_kq[kVtC];
  __shared__ int s_na[kVtC];
  __shared__ int s_pe[RP ? kVtT : 1];
  __shared__ int s_bad, s_pbad;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int G = p.Hv / p.Hk;
  const int n_units = p.L * p.B * p.Hk;
  const UnitSub us = xcd_unit_sub(blockIdx.x, G);
  if (us.unit >= n_units) return;
  const int hk = us.unit % p.Hk;
  const size_t lb = us.unit / p.Hk;
  const int l = static_cast<int>(lb / p.B);
  const int bb = static_cast<int>(lb % p.B);
  const int g = us.sub;
  const int hv = hk * G + g;
  const int T = p.T, C = p.C;
  const int K = KC > 0 ? KC : p.K;
  const int r = tid / TPR, h = tid % TPR;
  const bool lead = l == 0 && hk == 0 && g == 0;  // reports per-sequence errors once

  // this thread's slice of state row r
  floatx4 S[NQ];
  const size_t srow = ((lb * p.Hv + hv) * D + r) * static_cast<size_t>(D) + 4 * h;
#pragma unroll
  for (int m = 0; m < NQ; ++m) S[m] = *reinterpret_cast<const floatx4*>(p.S + srow + 4 * TPR * m);

  int pn = 0;
  if constexpr (RP) {
    const int v = p.prev_n_keep ? p.prev_n_keep[bb] : p.prev_n_all;
    pn = (v >= 0 && v <= p.pT) ? v : 0;
    if (pn != v && tid == 0 && p.dev_err && lead) atomicOr(p.dev_err, GDN_DEV_ERR_N_KEEP);
  }

  // ------------------------------------------ node structure (wave 0) --
  if (wave == 0) {
    const int t = lane;
    int pv = t - 1;
    bool bad = false;
    if (t < T && p.parent) {
      pv = p.parent[static_cast<size_t>(bb) * T + t];
      bad = pv < -1 || pv >= t;
      if (bad) pv = -1;
    }
    s_par[t] = t < T ? pv : -1;
    const unsigned long long anyb = __ballot(bad);
    if (lane == 0) s_bad = anyb != 0ull;
    wave_fence();
    // conv window of node t: the node, then its ancestors upward, then the
    // old conv rows (-1, -2, ...); entry K-1 is the node itself
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
      s_widx[t * KM + j] = w;
      if (j < K && t < T && p.conv_win && p.parent && lead)
        p.conv_win[(static_cast<size_t>(bb) * T + t) * K + j] = w;
    }
  }
  if constexpr (RP) {
    // wave 1: the previous accepted path, validated
    if (wave == 1) {
      int e = lane;
      bool bad = false;
      if (lane < pn) {
        if (p.prev_path) e = p.prev_path[static_cast<size_t>(bb) * p.pT + lane];
        bad = e < 0 || e >= p.pT;
      }
      s_pe[lane] = (lane < pn && !bad) ? e : 0;
      const unsigned long long anyb = __ballot(bad);
      if (lane == 0) s_pbad = anyb != 0ull;
    }
    __syncthreads();
    if (s_pbad) {
      if (tid == 0 && p.dev_err && lead) atomicOr(p.dev_err, GDN_DEV_ERR_PATH);
      pn = 0;
    }
    // the accepted steps' k, g and u, staged over the per-node arrays
    for (int e = tid; e < pn * D; e += NT) {
      const int i = e / D, c = e % D;
      const size_t te = lb * p.pT + s_pe[i];
      s_k[i][c] = p.ptk[(te * p.Hk + hk) * D + c];
      s_a[i][c] = p.ptg[(te * p.Hv + hv) * D + c];
      s_u[i][c] = p.ptu[(te * p.Hv + hv) * D + c];
    }
    __syncthreads();
    if (pn > 0) {
      for (int i = 0; i < pn; ++i) {
        const float ui = s_u[i][r];
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
          const floatx4 a4 = *reinterpret_cast<const floatx4*>(&s_a[i][4 * h + 4 * TPR * m]);
          const floatx4 k4 = *reinterpret_cast<const floatx4*>(&s_k[i][4 * h + 4 * TPR * m]);
          S[m] = S[m] * a4 + ui * k4;
        }
      }
#pragma unroll
      for (int m = 0; m < NQ; ++m)
        *reinterpret_cast<floatx4*>(p.S_out + srow + 4 * TPR * m) = S[m];
    }
    __syncthreads();  // staging consumed
  }

  // local channel lc in [q | k | v] of this head -> qkv channel
  auto chan = [&](int lc) {
    return lc < D ? hk * D + lc
                  : (lc < 2 * D ? p.Hk * D + hk * D + (lc - D) : 2 * p.Hk * D + hv * D + (lc - 2 * D));
  };
  {
    const float* cw = p.conv_w + static_cast<size_t>(l) * C * K;
    for (int e = tid; e < 3 * D * KM; e += NT) {
      const int lc = e / KM, j = e % KM;
      s_w[e] = j < K ? cw[static_cast<size_t>(chan(lc)) * K + j] : 0.f;
    }
    const TIn* ag = static_cast<const TIn*>(p.a);
    for (int e = tid; e < T * D; e += NT) {
      const int t = e / D, c = e % D;
      const size_t gi = ((lb * T + t) * p.Hv + hv) * D + c;
      const float av = ld_in(ag, gi);
      s_a[t][c] = av;
      p.tg[gi] = av;
    }
    for (int t = tid; t < T; t += NT)
      s_b[t] = ld_in(static_cast<const TIn*>(p.b), (lb * T + t) * p.Hv + hv);
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0 && p.dev_err) atomicOr(p.dev_err, GDN_DEV_ERR_PARENT);
    return;
  }

  const TIn* x = static_cast<const TIn*>(p.x) + lb * T * C;
  const TIn* cs = static_cast<const TIn*>(p.conv_state) + lb * (K - 1) * C;
  for (int c0 = 0; c0 < T; c0 += kVtC) {
    const int tc = T - c0 < kVtC ? T - c0 : kVtC;
    // ------------------------------------------------------ conv + SiLU --
    for (int it = tid; it < tc * NG; it += NT) {
      const int tl = it / NG, lc = (it % NG) * 4, t = c0 + tl;
      const int qc = chan(lc);
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j < K) {
          const int w = s_widx[t * KM + j];
          const TIn* src = w < 0 ? cs + static_cast<size_t>(K - 1 + w) * C + qc
                                 : x + static_cast<size_t>(w) * C + qc;
          const floatx4 xv = Quad<TIn>::load(src);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = fmaf(s_w[(lc + e) * KM + j], xv[e], acc[e]);
        }
      }
      if (p.silu) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = acc[e] * __builtin_amdgcn_rcpf(1.f + __expf(-acc[e]));
      }
      float* dst = lc < D ? &s_q[tl][lc] : (lc < 2 * D ? &s_k[t][lc - D] : &s_v[tl][lc - 2 * D]);
      *reinterpret_cast<floatx4*>(dst) = acc;
    }
    __syncthreads();
    // ------------------------------- L2 norms of q and k, wave per node --
    for (int tl = wave; tl < tc; tl += NWV) {
      const int t = c0 + tl;
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int m = 0; m < MPL; ++m) {
        const int c = lane + kWave * m;
        if (c < D) {
          sq = fmaf(s_q[tl][c], s_q[tl][c], sq);
          sk = fmaf(s_k[t][c], s_k[t][c], sk);
        }
      }
      sq = wave_total(sq);
      sk = wave_total(sk);
      const float rq = __builtin_amdgcn_rsqf(sq + p.eps), rk = __builtin_amdgcn_rsqf(sk + p.eps);
#pragma unroll
      for (int m = 0; m < MPL; ++m) {
        const int c = lane + kWave * m;
        if (c < D) {
          s_q[tl][c] *= rq;
          const float kn = s_k[t][c] * rk;
          s_k[t][c] = kn;
          if (g == 0) p.tk[((lb * T + t) * p.Hk + hk) * D + c] = kn;
        }
      }
    }
    __syncthreads();
    // ------------------------- path coefficients, wave per node, upward --
    for (int tl = wave; tl < tc; tl += NWV) {
      const int v = c0 + tl;
      float w[MPL], kv[MPL], qv[MPL];
      float kq = 0.f;
#pragma unroll
      for (int m = 0; m < MPL; ++m) {
        const int c = lane + kWave * m;
        const bool ok = c < D;
        w[m] = ok ? s_a[v][c] : 0.f;
        kv[m] = ok ? s_k[v][c] : 0.f;
        qv[m] = ok ? s_q[tl][c] : 0.f;
        kq = fmaf(kv[m], qv[m], kq);
      }
      int na = 0;
      for (int i = s_par[v]; i >= 0; i = s_par[i]) {
        float cc = 0.f, dd = 0.f;
#pragma unroll
        for (int m = 0; m < MPL; ++m) {
          const int c = lane + kWave * m;
          if (c < D) {
            const float kw = s_k[i][c] * w[m];
            cc = fmaf(kw, kv[m], cc);
            dd = fmaf(kw, qv[m], dd);
            w[m] *= s_a[i][c];
          }
        }
        cc = wave_total(cc);
        dd = wave_total(dd);
        if (lane == 0) {
          s_c[tl][na] = cc;
          s_d[tl][na] = dd;
          s_ai[tl][na] = i;
        }
        ++na;
      }
#pragma unroll
      for (int m = 0; m < MPL; ++m) {
        const int c = lane + kWave * m;
        if (c < D) {
          s_gk[tl][c] = w[m] * kv[m];
          s_gq[tl][c] = w[m] * qv[m];
        }
      }
      kq = wave_total(kq);
      if (lane == 0) {
        s_kq[tl] = kq;
        s_na[tl] = na;
      }
    }
    __syncthreads();
    // ------------------------------------------ the rows, node by node --
    for (int tl = 0; tl < tc; ++tl) {
      const int v = c0 + tl;
      float sd = 0.f, od = 0.f;
#pragma unroll
      for (int m = 0; m < NQ; ++m) {
        const floatx4 gk = *reinterpret_cast<const floatx4*>(&s_gk[tl][4 * h + 4 * TPR * m]);
        const floatx4 gq = *reinterpret_cast<const floatx4*>(&s_gq[tl][4 * h + 4 * TPR * m]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sd = fmaf(S[m][e], gk[e], sd);
          od = fmaf(S[m][e], gq[e], od);
        }
      }
      const int na = s_na[tl];
      for (int s = h; s < na; s += TPR) {
        const float ui = s_u[s_ai[tl][s]][r];
        sd = fmaf(ui, s_c[tl][s], sd);
        od = fmaf(ui, s_d[tl][s], od);
      }
      sd = group_sum<TPR>(sd);
      od = group_sum<TPR>(od);
      const float u = s_b[v] * (s_v[tl][r] - sd);
      const float ov = fmaf(u, s_kq[tl], od);
      if (h == 0) {
        s_u[v][r] = u;
        const size_t oi = ((lb * T + v) * p.Hv + hv) * D + r;
        p.tu[oi] = u;
        p.o[oi] = ov;
      }
      wave_fence();  // this row's u is read back by its own lanes
    }
    __syncthreads();  // the chunk arrays are rewritten next
  }
}

template <int D, int KC, typename TIn>
void launch_vgt_k(const VerifyArgs& a, bool rp, hipStream_t s, long long grid) {
  if (rp)
    hipLaunchKernelGGL((k_verify_vgt<D, KC, TIn, true>), dim3(grid), dim3(vgt_threads<D>()), 0, s, a);
  else
    hipLaunchKernelGGL((k_verify_vgt<D, KC, TIn, false>), dim3(grid), dim3(vgt_threads<D>()), 0, s, a);
}

template <int D, typename TIn>
void launch_vgt_d(const VerifyArgs& a, bool rp, hipStream_t s, long long grid) {
  if (a.K == 4)
    launch_vgt_k<D, 4, TIn>(a, rp, s, grid);
  else
    launch_vgt_k<D, 0, TIn>(a, rp, s, grid);
}

template <typename TIn>
hipError_t launch_vgt_t(const VerifyArgs& a, int d, hipStream_t s) {
  const bool rp = a.prev_n_keep || a.prev_n_all > 0;
  const int G = a.Hv / a.Hk;
  const int n_units = a.L * a.B * a.Hk;
  const long long grid = static_cast<long long>((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * G;
  if (grid > 0x7fffffffLL || a.T < 1 || a.T > kVtT || a.K < 1 || a.K > 8) return hipErrorInvalidValue;
  if (rp && (a.pT < 1 || a.pT > kVtT || !a.S_out || !a.ptu || !a.ptk || !a.ptg))
    return hipErrorInvalidValue;
  if (rp && !a.prev_n_keep && a.prev_n_all > a.pT) return hipErrorInvalidValue;
  switch (d) {
    case 32: launch_vgt_d<32, TIn>(a, rp, s, grid); break;
    case 64: launch_vgt_d<64, TIn>(a, rp, s, grid); break;
    case 128: launch_vgt_d<128, TIn>(a, rp, s, grid); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_vg_tree(const VerifyArgs& a, int dk, int dv, int dtype, hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  return dtype == 1 ? launch_vgt_t<uint16_t>(a, dk, s) : launch_vgt_t<float>(a, dk, s);
}

}  // namespace gdn
