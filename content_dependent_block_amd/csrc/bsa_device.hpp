// bsa_device.hpp -- device-side helpers shared by the gfx950 kernels:
// vector types, bf16 conversions, the MFMA instructions used, wave-level
// ballots.  Lane layouts were checked on gfx950: for the 16x16 MFMA shapes,
// operand slot (lane l, element i) of A pairs with slot (lane l', element i)
// of B when l / 16 == l' / 16, and the result C[m][n] sits in lane
// n + 16 * (m / 4), element m % 4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_bits;

constexpr int kWave = 64;
constexpr int kTile = 64;  // key block = key tile = query tile

__device__ __forceinline__ float bf16_to_f32(bf16_bits b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 f32_to_bf16(float f) {
  return static_cast<__bf16>(f);
}

__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(const bf16x8& a, const bf16x8& b,
                                                     const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x4_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// 16-byte global load / store helpers.
template <typename T>
__device__ __forceinline__ uint4 ld16(const T* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

}  // namespace bsa
