// coarse_score.hip -- Stage 1 scoring: s[i][beta] = q_i . repr_beta for every
// query and every block representative (nishantmodi.me
// "sparse-attention-triton-bench", section "Stage 1: coarse scoring": Q times
// the transposed block representatives, O(N * N/B) work).  Unscaled: a
// positive softmax scale would not change the ranking.
//
// Per (batch*head) this is a GEMM with M = n queries, N = n/64 blocks,
// K = d, run on MFMA.  A workgroup owns 64 queries (4 waves x 16) and walks
// the block representatives in tiles of 64, which it stages in LDS.
//   bf16 inputs: q is exact bf16; the float32 representative r is split into
//     three bf16 terms hi + mid + lo (each the bf16 rounding of what is left),
//     which carry r to about 24 significant bits, and the three products are
//     accumulated in fp32 by v_mfma_f32_16x16x32_bf16.  Without the split the
//     selection would differ from the exact one for a few percent of queries.
//   fp32 inputs: v_mfma_f32_16x16x4_f32 on the float32 values.
// Output: a float32 panel, one row of n/64 scores per query.  In the causal
// variant block tiles entirely after the query tile are skipped.
#include "bsa_device.hpp"
#include "bsa_launch.hpp"

namespace bsa {
namespace {

constexpr int kTerms = 3;

template <int D>
__global__ __launch_bounds__(256) void coarse_bf16_kernel(const bf16_bits* __restrict__ q,
                                                          const float* __restrict__ repr,
                                                          float* __restrict__ panel, int64_t row0,
                                                          int n, int causal) {
  constexpr int KS = D / 32;        // MFMA k-steps over d
  constexpr int PITCH = D + 8;      // bf16 elements per LDS row (16 B pad)
  __shared__ __bf16 rs[kTerms][kTile][PITCH];

  const int nb = n / kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t tile_row = row0 + static_cast<int64_t>(blockIdx.x) * kTile;  // first query row
  const int64_t bh = tile_row / n;
  const int i0 = static_cast<int>(tile_row % n);
  const int64_t prow_base = tile_row - row0;  // panel row of the tile's first query

  // A operand: this lane's query row, d = 8g + 32ks .. +7.
  bf16x8 qa[KS];
  {
    const bf16_bits* qr = q + (tile_row + wave * 16 + c16) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = as_bf16x8(ld16(qr + 32 * ks));
  }

  const float* rbase = repr + bh * static_cast<int64_t>(nb) * D;
  const int nbt_all = (nb + kTile - 1) / kTile;
  const int nbt = causal ? (i0 / kTile) / kTile + 1 : nbt_all;
  for (int bt = 0; bt < nbt; ++bt) {
    __syncthreads();
    // Stage 64 representatives as three bf16 terms.
    for (int c = tid; c < kTile * D / 4; c += 256) {
      const int r = c / (D / 4), col = (c % (D / 4)) * 4;
      const int beta = bt * kTile + r;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (beta < nb) x = *reinterpret_cast<const float4*>(rbase + static_cast<int64_t>(beta) * D + col);
      float v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int t = 0; t < kTerms; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 h = f32_to_bf16(v[e]);
          rs[t][r][col + e] = h;
          v[e] -= static_cast<float>(h);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int beta0 = bt * kTile + nt * 16;
      if (beta0 >= nb) break;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int t = 0; t < kTerms; ++t) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(&rs[t][nt * 16 + c16][8 * g + 32 * ks]);
          acc = mfma_16x16x32_bf16(qa[ks], b, acc);
        }
      }
      // lane holds C[query 4g + j][block c16]
      const int beta = beta0 + c16;
      if (beta < nb) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          panel[(prow_base + wave * 16 + 4 * g + j) * nb + beta] = acc[j];
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void coarse_f32_kernel(const float* __restrict__ q,
                                                         const float* __restrict__ repr,
                                                         float* __restrict__ panel, int64_t row0,
                                                         int n, int causal) {
  constexpr int KS = D / 4;     // MFMA k-steps; slot (ks, g) carries d = KS*g + ks
  constexpr int PITCH = D + 4;
  __shared__ float rs[kTile][PITCH];

  const int nb = n / kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t tile_row = row0 + static_cast<int64_t>(blockIdx.x) * kTile;
  const int64_t bh = tile_row / n;
  const int i0 = static_cast<int>(tile_row % n);
  const int64_t prow_base = tile_row - row0;

  float qa[KS];
  {
    const float* qr = q + (tile_row + wave * 16 + c16) * D + KS * g;
#pragma unroll
    for (int e = 0; e < KS; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(qr + e);
      qa[e] = x.x; qa[e + 1] = x.y; qa[e + 2] = x.z; qa[e + 3] = x.w;
    }
  }
  const float* rbase = repr + bh * static_cast<int64_t>(nb) * D;
  const int nbt_all = (nb + kTile - 1) / kTile;
  const int nbt = causal ? (i0 / kTile) / kTile + 1 : nbt_all;
  for (int bt = 0; bt < nbt; ++bt) {
    __syncthreads();
    for (int c = tid; c < kTile * D / 4; c += 256) {
      const int r = c / (D / 4), col = (c % (D / 4)) * 4;
      const int beta = bt * kTile + r;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (beta < nb) x = *reinterpret_cast<const float4*>(rbase + static_cast<int64_t>(beta) * D + col);
      *reinterpret_cast<float4*>(&rs[r][col]) = x;
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int beta0 = bt * kTile + nt * 16;
      if (beta0 >= nb) break;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* rr = &rs[nt * 16 + c16][KS * g];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma_16x16x4_f32(qa[ks], rr[ks], acc);
      const int beta = beta0 + c16;
      if (beta < nb) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          panel[(prow_base + wave * 16 + 4 * g + j) * nb + beta] = acc[j];
      }
    }
  }
}

}  // namespace

hipError_t launch_coarse_score(const void* q, const float* repr, float* panel, int64_t row0,
                               int64_t rows, int n, int d, bsa_dtype dtype, int causal,
                               hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(rows / kTile)), block(256);
  if (dtype == BSA_BF16) {
    const bf16_bits* qq = static_cast<const bf16_bits*>(q);
    if (d == 64)
      hipLaunchKernelGGL(coarse_bf16_kernel<64>, grid, block, 0, stream, qq, repr, panel, row0, n, causal);
    else
      hipLaunchKernelGGL(coarse_bf16_kernel<128>, grid, block, 0, stream, qq, repr, panel, row0, n, causal);
  } else {
    const float* qq = static_cast<const float*>(q);
    if (d == 64)
      hipLaunchKernelGGL(coarse_f32_kernel<64>, grid, block, 0, stream, qq, repr, panel, row0, n, causal);
    else
      hipLaunchKernelGGL(coarse_f32_kernel<128>, grid, block, 0, stream, qq, repr, panel, row0, n, causal);
  }
  return hipGetLastError();
}

}  // namespace bsa
