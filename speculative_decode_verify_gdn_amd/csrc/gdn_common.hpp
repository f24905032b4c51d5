// gdn_common.hpp -- device helpers shared by the gfx950 kernels of libgdnverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kWave = 64;  // CDNA wavefront width

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Split two fp32 values into packed bf16 high parts and bf16 residuals,
// x ~ hi + lo with |x - hi - lo| <= 2^-18 |x| (both roundings to nearest
// even).  Each pair takes one packed conversion for the highs and one for
// the residuals; the highs widen back exactly by a shift or a mask.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){a, b}, bf16x2));
  const float ra = a - __uint_as_float(h << 16);
  const float rb = b - __uint_as_float(h & 0xffff0000u);
  hi = h;
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){ra, rb}, bf16x2));
}

// The same for 8 values: hi and lo hold a[0..3] then b[0..3].  One
// conversion per value; it keeps fewer values live than the paired form
// below, which kernels near their register limit need.
__device__ __forceinline__ void split_bf16x8(const floatx4& a, const floatx4& b, bf16x8& hi,
                                             bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 ha = static_cast<__bf16>(a[e]);
    const __bf16 hb = static_cast<__bf16>(b[e]);
    hi[e] = ha;
    hi[e + 4] = hb;
    lo[e] = static_cast<__bf16>(a[e] - static_cast<float>(ha));
    lo[e + 4] = static_cast<__bf16>(b[e] - static_cast<float>(hb));
  }
}

// The same split by packed conversions of pairs (split_pair): bit-identical
// results in about half the instructions.
__device__ __forceinline__ void split_bf16x8_pk(const floatx4& a, const floatx4& b, bf16x8& hi,
                                                bf16x8& lo) {
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  split_pair(a[0], a[1], h0, l0);
  split_pair(a[2], a[3], h1, l1);
  split_pair(b[0], b[1], h2, l2);
  split_pair(b[2], b[3], h3, l3);
  hi = __builtin_bit_cast(bf16x8, (u32x4){h0, h1, h2, h3});
  lo = __builtin_bit_cast(bf16x8, (u32x4){l0, l1, l2, l3});
}

// fp32-accurate product on bf16 MFMA (16x16x32): acc += A B with each
// operand split hi + lo and the lo*lo term dropped (relative error ~1e-5).
__device__ __forceinline__ floatx4 mfma_bf16x3(const bf16x8& ahi, const bf16x8& alo,
                                               const bf16x8& bhi, const bf16x8& blo, floatx4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bhi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, blo, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bhi, acc, 0, 0, 0);
  return acc;
}

// Input element loads: fp32 as is, bf16 (raw uint16 bits) widened exactly.
__device__ __forceinline__ float ld_in(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld_in(const uint16_t* p, size_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// Sum over the 64 lanes of a wavefront; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Fold the blockIdx of a 1-D grid so that consecutive "slots" of the same
// unit land on the same XCD.  The hardware dispatches workgroup i to XCD
// i % 8; this returns (unit, sub) such that all `nsub` workgroups of one unit
// share an XCD (and its L2).  Grid size must be round_up(n_units, 8) * nsub.
struct UnitSub {
  int unit;
  int sub;
};
constexpr int kNumXcd = 8;
__device__ __forceinline__ UnitSub xcd_unit_sub(int bid, int nsub) {
  const int xcd = bid % kNumXcd;
  const int slot = bid / kNumXcd;
  UnitSub r;
  r.unit = (slot / nsub) * kNumXcd + xcd;
  r.sub = slot % nsub;
  return r;
}

}  // namespace gdn
