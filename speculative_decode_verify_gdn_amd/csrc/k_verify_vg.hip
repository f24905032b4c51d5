// k_verify_vg.hip -- verify of a chain of T <= 64 tokens through GDN layers
// whose decay gate acts per key channel, for gfx950.
//
// The GDN page's tape (s4) carries the decay gate either per v-head
// ([B,T,Hv]) or per v-head and key channel ([B,T,Hv,Dk]).  Under the second
// form the state decays column by column, and the delta rule (s2.1) reads
//   S <- S diag(a_t);  u_t = b_t (v_t - S k_t);  S <- S + u_t k_t^T;  o_t = S q_t.
// The chunked WY form of the scalar kernels would need ratios of per-channel
// gate products, which overflow or underflow for small gates over a chunk,
// so this kernel runs the recurrence itself: the state stays in registers
// and each token costs four multiply-adds per state element.
//
// One workgroup per (layer, seq, v-head), 512 threads for 128-dim heads and
// 256 otherwise.  Thread (row r, part h)
// owns columns [h*CPT, (h+1)*CPT) of state row r (TPR threads per row); the
// row's dot products are reduced across those TPR lanes.  Tokens go through
// in chunks of 16: all threads compute the chunk's conv + SiLU of the head's
// q, k and v channels into LDS, one wave per token takes the q / k norms,
// then every thread steps its row slice through the chunk.  S is read once
// and not written (it stays the snapshot), except by the prefill, which sets
// S_out, passes no tape, and gets the state after the last token written
// back in place.

#include "gdn_common.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

constexpr int kVgTC = 16;  // tokens per staged chunk

// 512 threads for 128-dim heads (four per state row keeps the row slice at
// 32 registers and four waves per SIMD), 256 otherwise.
template <int D>
constexpr int vg_threads() {
  return D == 128 ? 512 : 256;
}

template <int D, typename TIn>
__global__ __launch_bounds__(vg_threads<D>()) void k_verify_vg(VerifyArgs p) {
  constexpr int kVgNT = vg_threads<D>();
  constexpr int TPR = kVgNT / D;  // threads per state row
  constexpr int CPT = D / TPR;    // columns per thread
  static_assert(CPT % 4 == 0, "float4 columns");
  constexpr int NWV = kVgNT / kWave;
  __shared__ __align__(16) float s_q[kVgTC][D];
  __shared__ __align__(16) float s_k[kVgTC][D];
  __shared__ __align__(16) float s_v[kVgTC][D];
  __shared__ __align__(16) float s_a[kVgTC][D];
  __shared__ float s_b[kVgTC];

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
  const int g = us.sub;
  const int hv = hk * G + g;
  const int T = p.T, K = p.K, C = p.C;
  const int r = tid / TPR, h = tid % TPR, c0 = h * CPT;

  // this thread's slice of state row r
  floatx4 S[CPT / 4];
  const float* Srow = p.S + ((lb * p.Hv + hv) * D + r) * static_cast<size_t>(D) + c0;
#pragma unroll
  for (int j = 0; j < CPT / 4; ++j) S[j] = reinterpret_cast<const floatx4*>(Srow)[j];

  const TIn* x = static_cast<const TIn*>(p.x) + lb * T * C;
  const TIn* cs = static_cast<const TIn*>(p.conv_state) + lb * (K - 1) * C;
  const float* cw = p.conv_w + static_cast<size_t>(l) * C * K;
  // local channel ch in [q | k | v] of this head -> qkv channel
  auto chan = [&](int ch) {
    return ch < D ? hk * D + ch
                  : (ch < 2 * D ? p.Hk * D + hk * D + (ch - D) : 2 * p.Hk * D + hv * D + (ch - 2 * D));
  };

  for (int t0 = 0; t0 < T; t0 += kVgTC) {
    const int tc = T - t0 < kVgTC ? T - t0 : kVgTC;
    __syncthreads();  // the previous chunk's LDS has been consumed
    // conv (+ SiLU) of the head's 3D channels over the chunk's tokens; the
    // window of token t is rows t-K+1 .. t of [conv_state; x]
    // the channel's K-1 + tc source rows are loaded together (independent
    // loads, clamped to valid rows), then convolved from registers
    constexpr int XR = kVgTC + 7;
    for (int ch = tid; ch < 3 * D; ch += kVgNT) {
      const int qc = chan(ch);
      float w[8], xr[XR];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = j < K ? cw[static_cast<size_t>(qc) * K + j] : 0.f;
#pragma unroll
      for (int e = 0; e < XR; ++e) {
        int s = t0 + e - (K - 1);  // source row of window entry e
        s = s < T ? s : T - 1;
        xr[e] = s < 0 ? ld_in(cs, static_cast<size_t>(K - 1 + s) * C + qc)
                      : ld_in(x, static_cast<size_t>(s) * C + qc);
      }
#pragma unroll
      for (int t = 0; t < kVgTC; ++t) {
        if (t < tc) {
          float acc = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j < K) acc = fmaf(w[j], xr[t + j], acc);
          if (p.silu) acc = acc / (1.f + __expf(-acc));
          float* dst = ch < D ? &s_q[t][ch] : (ch < 2 * D ? &s_k[t][ch - D] : &s_v[t][ch - 2 * D]);
          *dst = acc;
        }
      }
    }
    // per-channel decay and write strength of the chunk's tokens
    for (int e = tid; e < tc * D; e += kVgNT) {
      const int t = e / D, c = e % D;
      s_a[t][c] = ld_in(static_cast<const TIn*>(p.a), ((lb * T + t0 + t) * p.Hv + hv) * D + c);
    }
    if (tid < tc) s_b[tid] = ld_in(static_cast<const TIn*>(p.b), (lb * T + t0 + tid) * p.Hv + hv);
    __syncthreads();
    // L2 norms of q and k, one wave per token
    for (int t = wave; t < tc; t += NWV) {
      float sq = 0.f, sk = 0.f;
      for (int c = lane; c < D; c += kWave) {
        sq = fmaf(s_q[t][c], s_q[t][c], sq);
        sk = fmaf(s_k[t][c], s_k[t][c], sk);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        sq += __shfl_xor(sq, off, kWave);
        sk += __shfl_xor(sk, off, kWave);
      }
      const float rq = __builtin_amdgcn_rsqf(sq + p.eps), rk = __builtin_amdgcn_rsqf(sk + p.eps);
      for (int c = lane; c < D; c += kWave) {
        s_q[t][c] *= rq;
        const float kn = s_k[t][c] * rk;
        s_k[t][c] = kn;
        if (p.tk && g == 0) p.tk[((lb * T + t0 + t) * p.Hk + hk) * D + c] = kn;
        if (p.tg) p.tg[((lb * T + t0 + t) * p.Hv + hv) * D + c] = s_a[t][c];
      }
    }
    __syncthreads();
    // the recurrence over the chunk, on this thread's row slice
    for (int t = 0; t < tc; ++t) {
      const floatx4* ka = reinterpret_cast<const floatx4*>(&s_k[t][c0]);
      const floatx4* qa = reinterpret_cast<const floatx4*>(&s_q[t][c0]);
      const floatx4* aa = reinterpret_cast<const floatx4*>(&s_a[t][c0]);
      float sd = 0.f;
#pragma unroll
      for (int j = 0; j < CPT / 4; ++j) {
        S[j] = S[j] * aa[j];
        const floatx4 kv = ka[j];
        sd = fmaf(S[j][0], kv[0], fmaf(S[j][1], kv[1], fmaf(S[j][2], kv[2], fmaf(S[j][3], kv[3], sd))));
      }
#pragma unroll
      for (int off = TPR / 2; off >= 1; off >>= 1) sd += __shfl_xor(sd, off, kWave);
      const float u = s_b[t] * (s_v[t][r] - sd);
      float od = 0.f;
#pragma unroll
      for (int j = 0; j < CPT / 4; ++j) {
        S[j] += u * ka[j];
        const floatx4 qv = qa[j];
        od = fmaf(S[j][0], qv[0], fmaf(S[j][1], qv[1], fmaf(S[j][2], qv[2], fmaf(S[j][3], qv[3], od))));
      }
#pragma unroll
      for (int off = TPR / 2; off >= 1; off >>= 1) od += __shfl_xor(od, off, kWave);
      if (h == 0) {
        const size_t oi = ((lb * T + t0 + t) * p.Hv + hv) * D + r;
        if (p.tu) p.tu[oi] = u;
        p.o[oi] = od;
      }
    }
  }
  // committing (prefill): the state after the last token goes back in place
  if (p.S_out) {
    float* Sw = p.S_out + ((lb * p.Hv + hv) * D + r) * static_cast<size_t>(D) + c0;
#pragma unroll
    for (int j = 0; j < CPT / 4; ++j) reinterpret_cast<floatx4*>(Sw)[j] = S[j];
  }
}

template <typename TIn>
hipError_t launch_vg_t(const VerifyArgs& a, int d, hipStream_t s) {
  const int G = a.Hv / a.Hk;
  const int n_units = a.L * a.B * a.Hk;
  const long long grid = static_cast<long long>((n_units + kNumXcd - 1) / kNumXcd) * kNumXcd * G;
  // verify writes a tape of T entries (T <= 64); committing (S_out set, no
  // tape) takes any T
  if (grid > 0x7fffffffLL || (a.T > 64 && !a.S_out) || a.K > 8) return hipErrorInvalidValue;
  switch (d) {
    case 32: hipLaunchKernelGGL((k_verify_vg<32, TIn>), dim3(grid), dim3(vg_threads<32>()), 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_verify_vg<64, TIn>), dim3(grid), dim3(vg_threads<64>()), 0, s, a); break;
    case 128: hipLaunchKernelGGL((k_verify_vg<128, TIn>), dim3(grid), dim3(vg_threads<128>()), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_vg(const VerifyArgs& a, int dk, int dv, int dtype, hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  return dtype == 1 ? launch_vg_t<uint16_t>(a, dk, s) : launch_vg_t<float>(a, dk, s);
}

}  // namespace gdn
