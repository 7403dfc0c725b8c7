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

// Maximum and sum of x over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one
// MFMA output column), with the gfx950 permlane swaps: called with the same
// register as both operands, a swap returns the lane's own value and its
// partner's (in an order that depends on the lane), so one max or add of the
// two results reduces over the pair without a select.
__device__ __forceinline__ float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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

// Sequences of different lengths.  The rows of a head hold one or more
// sequences one after the other, each padded with zero rows to whole 64-row
// blocks.  Entry beta of the block table describes block beta of that layout
// (the same for every head): {first block of its sequence, one past the
// sequence's last block, keys of the block that exist (1 .. 64), first caller
// row of the block}.  A NULL table means one sequence of n / 64 whole blocks
// per head.  Selections hold block numbers relative to the sequence's first
// block.
struct RowBlocks {
  int lo, hi;  // candidate blocks [lo, hi) of the row's head
  int own;     // the row's own block
};

__device__ __forceinline__ RowBlocks row_blocks(const int4* __restrict__ seqtab, int64_t row, int n,
                                                int causal) {
  RowBlocks r;
  r.own = static_cast<int>(row % n) / kTile;
  r.lo = 0;
  r.hi = n / kTile;
  if (seqtab) {
    const int4 e = seqtab[r.own];
    r.lo = e.x;
    r.hi = e.y;
  }
  if (causal) r.hi = r.own + 1;
  return r;
}

// The head-level block of selection entry `sel`, or -1 when the entry does
// not count (padding, outside the row's sequence, after its own block in the
// causal variant).
__device__ __forceinline__ int sel_block(int sel, const RowBlocks& r) {
  return (sel >= 0 && sel < r.hi - r.lo) ? r.lo + sel : -1;
}

// Keys of block beta that exist.
__device__ __forceinline__ int block_keys(const int4* __restrict__ seqtab, int beta) {
  return seqtab ? seqtab[beta].z : kTile;
}

}  // namespace bsa
