// coarse_score.hip -- Stage 1 scoring: s[i][beta] = q_i . repr_beta for every
// query and every block representative (nishantmodi.me
// "sparse-attention-triton-bench", section "Stage 1: coarse scoring": Q times
// the transposed block representatives, O(N * N/B) work).  Unscaled: a
// positive softmax scale would not change the ranking.
//
// Per (batch*head) this is a GEMM with M = n/64 blocks, N = n queries,
// K = d (C = R Q^T), run on MFMA.  A workgroup owns 64 queries (4 waves x 16)
// and walks the block representatives in tiles of 64, which it stages in LDS.
//   bf16 inputs: q is exact bf16; the float32 representative r is split into
//     three bf16 terms hi + mid + lo (each the bf16 rounding of what is left),
//     which carry r to about 24 significant bits, and the three products are
//     accumulated in fp32 by v_mfma_f32_16x16x32_bf16.  Without the split the
//     selection would differ from the exact one for a few percent of queries.
//   fp32 inputs: v_mfma_f32_16x16x4_f32 on the float32 values.
// In the C = R Q^T orientation lane l holds, for query l%16 of its wave, the
// scores of blocks 4*(l/16) + j of each 16-block tile.  In the causal variant
// block tiles entirely after the query tile are skipped.
//
// Two sinks for the scores:
//   panel mode: the float32 panel, block-major (panel[beta][row]), 16 lanes
//     storing 64 contiguous bytes of one block row.
//   select mode (k <= 32, the path bsa_forward takes): the scores never leave
//     the chip.  Each lane offers its scores, in ascending block order, to an
//     exact register top-KL list (topk_list.hpp, KL >= k); the query's answer
//     is contained in the union of its 4 lanes' lists, from which k_eff
//     rounds of a cross-lane tournament take it in rank order.  It is written
//     in ascending block order (topk_select.hip states the selection
//     semantics).
// Workgroups are issued XCD-major: consecutive workgroup ids go round-robin
// over the 8 XCDs, so tile t runs on XCD t / (tiles / 8) and each XCD's L2
// sees the representatives of as few heads as possible; in the causal
// variant each XCD takes its tiles heaviest first.
#include "bsa_device.hpp"
#include "bsa_launch.hpp"
#include "topk_list.hpp"

namespace bsa {
namespace {

constexpr int kTerms = 3;

__device__ __forceinline__ int64_t xcd_tile(int causal) {
  const int64_t nwg = gridDim.x, bid = blockIdx.x;
  if (nwg % 8 != 0) return bid;
  const int64_t per = nwg / 8, local = bid / 8;
  return (bid % 8) * per + (causal ? per - 1 - local : local);
}

// Is (va, ba) ranked above (vb, bb)?  Higher score first, then lower block.
__device__ __forceinline__ bool ranks_above(float va, int ba, float vb, int bb) {
  return va > vb || (va == vb && ba < bb);
}

// Consumer of the score tiles of one lane (query c16 of the wave; acc[j] is
// the score of block beta0 + j).
template <int KL>
struct Sink {
  TopList<KL> list;
  __device__ __forceinline__ void init() { list.init(); }
  __device__ __forceinline__ void take(const f32x4& acc, int beta0, int nb, int nvalid, int forced,
                                       float* __restrict__ panel, int64_t prows, int64_t prow) {
    if constexpr (KL == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (beta0 + j < nb) panel[static_cast<int64_t>(beta0 + j) * prows + prow] = acc[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int beta = beta0 + j;
        float x = beta == forced ? INFINITY : acc[j];
        x = beta < nvalid ? x : -INFINITY;
        list.offer(x, beta);
      }
    }
  }
  // Merge the 4 lists of each query and write its selection: k_eff rounds of
  // a 4-lane tournament between the lists' heads; the winner's lane drops
  // its head.  sel: LDS [4 waves][KL][16] receives the winners in rank order.
  __device__ __forceinline__ void finish(int* sel, int wave, int g, int c16, int keff, int topk,
                                         int32_t* __restrict__ dst) {
    if constexpr (KL > 0) {
      int* ws = sel + wave * KL * 16;
      for (int t = 0; t < keff; ++t) {
        float mv = list.v[0];
        int mb = list.b[0];
#pragma unroll
        for (int m = 16; m <= 32; m *= 2) {
          const float ov = __shfl_xor(mv, m);
          const int ob = __shfl_xor(mb, m);
          const bool take = ranks_above(ov, ob, mv, mb);
          mv = take ? ov : mv;
          mb = take ? ob : mb;
        }
        if (list.b[0] == mb) {
#pragma unroll
          for (int j = 0; j + 1 < KL; ++j) {
            list.v[j] = list.v[j + 1];
            list.b[j] = list.b[j + 1];
          }
          list.v[KL - 1] = -INFINITY;
          list.b[KL - 1] = -1;
        }
        if (g == 0) ws[t * 16 + c16] = mb;
      }
      __syncthreads();
      int b[KL];
#pragma unroll
      for (int u = 0; u < KL; ++u) b[u] = u < keff ? ws[u * 16 + c16] : 0x7fffffff;
#pragma unroll
      for (int t0 = 0; t0 < KL; t0 += 4) {
        const int t = t0 + g;
        if (t < keff) {
          int me = b[t0];
#pragma unroll
          for (int e = 1; e < 4; ++e) me = g == e ? b[t0 + e] : me;
          int pos = 0;
#pragma unroll
          for (int u = 0; u < KL; ++u) pos += b[u] < me ? 1 : 0;
          dst[pos] = me;
        }
      }
      for (int t = keff + g; t < topk; t += 4) dst[t] = -1;
    }
  }
};

// Panel rows: prows = rows of the chunk; panel[beta * prows + prow].
template <int D, int KL>
__global__ __launch_bounds__(256) void coarse_bf16_kernel(const bf16_bits* __restrict__ q,
                                                          const float* __restrict__ repr,
                                                          float* __restrict__ panel,
                                                          int32_t* __restrict__ idx, int64_t row0,
                                                          int64_t prows, int n, int topk, int causal) {
  constexpr int KS = D / 32;        // MFMA k-steps over d
  constexpr int PITCH = D + 8;      // bf16 elements per LDS row (16 B pad)
  __shared__ __bf16 rs[kTerms][kTile][PITCH];
  __shared__ int sel[4][KL > 0 ? KL : 1][16];

  const int nb = n / kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t tile_row = row0 + xcd_tile(causal) * kTile;  // first query row
  const int64_t bh = tile_row / n;
  const int i0 = static_cast<int>(tile_row % n);
  const int64_t qrow = tile_row + wave * 16 + c16;  // this lane's query
  const int64_t prow = qrow - row0;

  // B operand: this lane's query row, d = 8g + 32ks .. +7.
  bf16x8 qb[KS];
  {
    const bf16_bits* qr = q + qrow * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = as_bf16x8(ld16(qr + 32 * ks));
  }

  const float* rbase = repr + bh * static_cast<int64_t>(nb) * D;
  const int nbt_all = (nb + kTile - 1) / kTile;
  const int nbt = causal ? (i0 / kTile) / kTile + 1 : nbt_all;
  const int qblk = i0 / kTile;  // query block of all 64 rows
  const int nvalid = causal ? qblk + 1 : nb;
  const int forced = causal ? qblk : -1;
  Sink<KL> sink;
  sink.init();
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
    for (int mt = 0; mt < 4; ++mt) {
      if (bt * kTile + mt * 16 >= nb) break;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int t = 0; t < kTerms; ++t) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&rs[t][mt * 16 + c16][8 * g + 32 * ks]);
          acc = mfma_16x16x32_bf16(a, qb[ks], acc);
        }
      }
      // lane holds C[block 4g + j][query c16]
      sink.take(acc, bt * kTile + mt * 16 + 4 * g, nb, nvalid, forced, panel, prows, prow);
    }
  }
  if constexpr (KL > 0) {
    const int keff = topk < nvalid ? topk : nvalid;
    sink.finish(&sel[0][0][0], wave, g, c16, keff, topk, idx + qrow * topk);
  }
}

template <int D, int KL>
__global__ __launch_bounds__(256) void coarse_f32_kernel(const float* __restrict__ q,
                                                         const float* __restrict__ repr,
                                                         float* __restrict__ panel,
                                                         int32_t* __restrict__ idx, int64_t row0,
                                                         int64_t prows, int n, int topk, int causal) {
  constexpr int KS = D / 4;     // MFMA k-steps; slot (ks, g) carries d = KS*g + ks
  constexpr int PITCH = D + 4;
  __shared__ float rs[kTile][PITCH];
  __shared__ int sel[4][KL > 0 ? KL : 1][16];

  const int nb = n / kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t tile_row = row0 + xcd_tile(causal) * kTile;
  const int64_t bh = tile_row / n;
  const int i0 = static_cast<int>(tile_row % n);
  const int64_t qrow = tile_row + wave * 16 + c16;
  const int64_t prow = qrow - row0;

  float qf[KS];
  {
    const float* qr = q + qrow * D + KS * g;
#pragma unroll
    for (int e = 0; e < KS; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(qr + e);
      qf[e] = x.x; qf[e + 1] = x.y; qf[e + 2] = x.z; qf[e + 3] = x.w;
    }
  }
  const float* rbase = repr + bh * static_cast<int64_t>(nb) * D;
  const int nbt_all = (nb + kTile - 1) / kTile;
  const int nbt = causal ? (i0 / kTile) / kTile + 1 : nbt_all;
  const int qblk = i0 / kTile;
  const int nvalid = causal ? qblk + 1 : nb;
  const int forced = causal ? qblk : -1;
  Sink<KL> sink;
  sink.init();
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
    for (int mt = 0; mt < 4; ++mt) {
      if (bt * kTile + mt * 16 >= nb) break;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* rr = &rs[mt * 16 + c16][KS * g];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma_16x16x4_f32(rr[ks], qf[ks], acc);
      sink.take(acc, bt * kTile + mt * 16 + 4 * g, nb, nvalid, forced, panel, prows, prow);
    }
  }
  if constexpr (KL > 0) {
    const int keff = topk < nvalid ? topk : nvalid;
    sink.finish(&sel[0][0][0], wave, g, c16, keff, topk, idx + qrow * topk);
  }
}

template <int D, int KL>
void launch_kl(const void* q, const float* repr, float* panel, int32_t* idx, int64_t row0,
               int64_t rows, int n, bsa_dtype dtype, int topk, int causal, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(rows / kTile)), block(256);
  if (dtype == BSA_BF16)
    hipLaunchKernelGGL((coarse_bf16_kernel<D, KL>), grid, block, 0, stream,
                       static_cast<const bf16_bits*>(q), repr, panel, idx, row0, rows, n, topk, causal);
  else
    hipLaunchKernelGGL((coarse_f32_kernel<D, KL>), grid, block, 0, stream,
                       static_cast<const float*>(q), repr, panel, idx, row0, rows, n, topk, causal);
}

template <int KL>
void launch_d(const void* q, const float* repr, float* panel, int32_t* idx, int64_t row0,
              int64_t rows, int n, int d, bsa_dtype dtype, int topk, int causal, hipStream_t stream) {
  if (d == 64) launch_kl<64, KL>(q, repr, panel, idx, row0, rows, n, dtype, topk, causal, stream);
  else launch_kl<128, KL>(q, repr, panel, idx, row0, rows, n, dtype, topk, causal, stream);
}

}  // namespace

hipError_t launch_coarse_score(const void* q, const float* repr, float* panel, int64_t row0,
                               int64_t rows, int n, int d, bsa_dtype dtype, int causal,
                               hipStream_t stream) {
  launch_d<0>(q, repr, panel, nullptr, row0, rows, n, d, dtype, 1, causal, stream);
  return hipGetLastError();
}

hipError_t launch_coarse_select(const void* q, const float* repr, int32_t* idx, int64_t rows,
                                int n, int d, bsa_dtype dtype, int topk, int causal,
                                hipStream_t stream) {
  if (topk <= 8) launch_d<8>(q, repr, nullptr, idx, 0, rows, n, d, dtype, topk, causal, stream);
  else if (topk <= 16) launch_d<16>(q, repr, nullptr, idx, 0, rows, n, d, dtype, topk, causal, stream);
  else launch_d<32>(q, repr, nullptr, idx, 0, rows, n, d, dtype, topk, causal, stream);
  return hipGetLastError();
}

}  // namespace bsa
