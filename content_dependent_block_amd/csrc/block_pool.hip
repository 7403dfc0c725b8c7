// block_pool.hip -- Stage 1 pooling: each 64-key block is reduced to its mean
// (nishantmodi.me "sparse-attention-triton-bench", section "Stage 1: coarse
// scoring": a representative per key block, by mean-pooling its keys).
//
// One wavefront per block.  Every lane loads 16 bytes per row chunk, so one
// load instruction of the wave covers 64 * 16 B = 1 KiB of contiguous keys;
// lanes that share a column chunk are then reduced with xor shuffles.  The
// kernel reads K exactly once and writes the float32 representatives, so it is
// bound by HBM bandwidth.
//
// When a sequence's length is not a multiple of 64 its keys come padded with
// zero rows to whole blocks, and its last block is the mean of the keys that
// exist (the sum over the padded block, divided by their count, which the
// block table gives).
//
// Optionally it also writes each representative r as three bfloat16 terms
// hi + mid + lo (hi = bf16(r), mid = bf16(r - hi), lo = bf16(r - hi - mid)),
// laid out as one plane per term and head, split[bh][term][beta][d], the form
// the fused scoring kernel feeds to the bf16 MFMA (coarse_score.hip explains
// the split), and the 2-norm of each block's hi term (rounded up), whose
// largest value over a head bounds that kernel's hi-only first pass error.
#include "bsa_device.hpp"
#include "bsa_launch.hpp"

namespace bsa {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void block_pool_kernel(const T* __restrict__ k,
                                                         float* __restrict__ repr,
                                                         bf16_bits* __restrict__ split,
                                                         float* __restrict__ hinorm,
                                                         int64_t total_blocks, int nb,
                                                         const int4* __restrict__ seqtab) {
  constexpr int E = 16 / sizeof(T);     // elements per 16-byte chunk
  constexpr int LPR = D / E;            // lanes per key row
  constexpr int RPL = kWave / LPR;      // rows per wave-wide load
  constexpr int ITERS = kTile / RPL;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (blk >= total_blocks) return;
  const int c = lane % LPR;
  const int ro = lane / LPR;
  const T* base = k + (blk * kTile + ro) * D + c * E;

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const uint4 u = ld16(base + static_cast<int64_t>(it) * RPL * D);
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(w[e] << 16);
        acc[2 * e + 1] += __uint_as_float(w[e] & 0xFFFF0000u);
      }
    } else {
      acc[0] += __uint_as_float(u.x);
      acc[1] += __uint_as_float(u.y);
      acc[2] += __uint_as_float(u.z);
      acc[3] += __uint_as_float(u.w);
    }
  }
#pragma unroll
  for (int s = LPR; s < kWave; s <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += __shfl_xor(acc[e], s);
  }
  if (ro == 0) {
    const int keys = block_keys(seqtab, static_cast<int>(blk % nb));
    if (keys < kTile) {  // a sequence's partial last block: mean of the keys that exist
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = acc[e] / static_cast<float>(keys);
    } else {
      constexpr float inv = 1.0f / kTile;  // exact: a power of two
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] *= inv;
    }
    if (repr) {
      float* dst = repr + blk * D + c * E;
#pragma unroll
      for (int e = 0; e < E; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
    }
    if (split) {
      // E consecutive d per lane; the planes of one head are nb * D apart.
      const int64_t bhi = blk / nb;
      bf16_bits* dst = split + (blk + 2 * bhi * nb) * D + c * E;
      float ss = 0.f;  // sum of squares of this lane's hi elements
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        uint32_t w[E / 2];
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          const __bf16 h0 = f32_to_bf16(acc[e]), h1 = f32_to_bf16(acc[e + 1]);
          if (t == 0) {
            ss = __builtin_fmaf(static_cast<float>(h0), static_cast<float>(h0), ss);
            ss = __builtin_fmaf(static_cast<float>(h1), static_cast<float>(h1), ss);
          }
          acc[e] -= static_cast<float>(h0);
          acc[e + 1] -= static_cast<float>(h1);
          w[e / 2] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
                     (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
        }
        if constexpr (E == 8) {
          *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(t) * nb * D) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
          *reinterpret_cast<uint2*>(dst + static_cast<int64_t>(t) * nb * D) = make_uint2(w[0], w[1]);
        }
      }
      // the row's LPR lanes (all with ro == 0) add their parts; rounded up by
      // 2^-16, more than the relative error of the fp32 sum and square root
#pragma unroll
      for (int s = 1; s < LPR; s <<= 1) ss += __shfl_xor(ss, s);
      if (c == 0) hinorm[blk] = __builtin_sqrtf(ss) * (1.0f + 0x1.0p-16f);
    }
  }
}

template <typename T, int D>
hipError_t launch(const void* k, float* repr, bf16_bits* split, int64_t blocks, int nb,
                  const int4* seqtab, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((blocks + 3) / 4));
  float* hinorm = split ? split_norms(split, blocks / nb, nb, D) : nullptr;
  hipLaunchKernelGGL((block_pool_kernel<T, D>), grid, dim3(256), 0, s,
                     static_cast<const T*>(k), repr, split, hinorm, blocks, nb, seqtab);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_pool(const void* k, float* repr, uint16_t* split, int64_t bh, int n, int d,
                             bsa_dtype dtype, hipStream_t stream, const int4* seqtab) {
  const int nb = n / kTile;
  const int64_t blocks = bh * nb;
  if (dtype == BSA_BF16) {
    return d == 64 ? launch<bf16_bits, 64>(k, repr, split, blocks, nb, seqtab, stream)
                   : launch<bf16_bits, 128>(k, repr, split, blocks, nb, seqtab, stream);
  }
  return d == 64 ? launch<float, 64>(k, repr, split, blocks, nb, seqtab, stream)
                 : launch<float, 128>(k, repr, split, blocks, nb, seqtab, stream);
}

}  // namespace bsa
