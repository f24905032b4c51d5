// gdn_common.hpp -- device helpers shared by the gfx950 kernels of libgdnverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kWave = 64;  // CDNA wavefront width

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes

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
