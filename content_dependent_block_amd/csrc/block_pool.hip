// block_pool.hip -- Stage 1 pooling: each 64-key block is reduced to its mean
// (nishantmodi.me "sparse-attention-triton-bench", section "Stage 1: coarse
// scoring": a representative per key block, by mean-pooling its keys).
//
// One wavefront per block.  Every lane loads 16 bytes per row chunk, so one
// load instruction of the wave covers 64 * 16 B = 1 KiB of contiguous keys;
// lanes that share a column chunk are then reduced with xor shuffles.  The
// kernel reads K exactly once and writes the float32 representatives, so it is
// bound by HBM bandwidth.
#include "bsa_device.hpp"
#include "bsa_launch.hpp"

namespace bsa {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void block_pool_kernel(const T* __restrict__ k,
                                                         float* __restrict__ repr,
                                                         int64_t total_blocks) {
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
    float* dst = repr + blk * D + c * E;
    constexpr float inv = 1.0f / kTile;  // exact: a power of two
#pragma unroll
    for (int e = 0; e < E; e += 4)
      *reinterpret_cast<float4*>(dst + e) =
          make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
  }
}

template <typename T, int D>
hipError_t launch(const void* k, float* repr, int64_t blocks, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((blocks + 3) / 4));
  hipLaunchKernelGGL((block_pool_kernel<T, D>), grid, dim3(256), 0, s,
                     static_cast<const T*>(k), repr, blocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_pool(const void* k, float* repr, int64_t bh, int n, int d,
                             bsa_dtype dtype, hipStream_t stream) {
  const int64_t blocks = bh * (n / kTile);
  if (dtype == BSA_BF16) {
    return d == 64 ? launch<bf16_bits, 64>(k, repr, blocks, stream)
                   : launch<bf16_bits, 128>(k, repr, blocks, stream);
  }
  return d == 64 ? launch<float, 64>(k, repr, blocks, stream)
                 : launch<float, 128>(k, repr, blocks, stream);
}

}  // namespace bsa
