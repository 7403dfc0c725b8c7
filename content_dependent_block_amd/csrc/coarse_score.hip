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
// The panel kernel (bsa_coarse_score, and the panel strategy of bsa_forward)
// writes the float32 scores block-major, panel[beta][row], 16 lanes storing
// 64 contiguous bytes of one block row.
//
// The select kernel (bsa_forward, k <= 32) never stores a score.  It walks
// the representatives twice:
//   pass 1: every lane keeps the maximum of each of its score groups, group =
//     beta mod G with G = 64 * GM (16 * GM groups per lane, the 4 lanes of a
//     query hold them all).  tau = the k_eff-th largest of the G group maxima
//     (each lane sorts its own; two pairwise bitonic merges between the
//     query's 4 lanes, over the gfx950 permlane swaps, give all 4 the top).
//     The k_eff groups whose maxima are >= tau each hold a score >= tau, so at
//     least k_eff scores are >= tau, and every score of the answer is >= tau.
//     For bf16 inputs pass 1 multiplies only the hi term of the split, at a
//     third of the MFMA and LDS work, and each group maximum enters less
//     (2^-8 + 2^-13) |q|_2 max |hi|_2 over the head's blocks (hi is r rounded
//     to 8 significant bits; Cauchy-Schwarz; the norms come from block_pool):
//     a lower bound of the group's largest exact score, which keeps tau a
//     bound for the exact scores.
//   pass 2: the same scores again; those >= tau (typically k + a few) are
//     appended to the lane's LDS slots in ascending block order.
//   The lane reads its slots into registers and sorts a copy of their
//     scores; two pairwise merges between the query's 4 lanes give each the
//     query's top scores, so T = the k_eff-th largest candidate.  The answer
//     is every candidate above T plus the lowest-block ties at T; the 4 lanes
//     put it in an LDS row, and each sorts the row's block ids and writes its
//     quarter of the output in ascending block order.  Because the answer is
//     ranked from pass 2's scores alone and pass 2 checks it holds >= k_eff
//     candidates, the result is exact.
//   A workgroup in which some lane has more candidates than slots walks
//     pass 2 again with tau raised to the k_eff-th largest candidate its lanes
//     kept; one in which that also overflows (or that has fewer than k_eff
//     candidates) redoes the walk offering every score to exact register
//     top-KL lists (topk_list.hpp) merged the same way: the same answer,
//     slower.
// topk_select.hip states the selection semantics.
//
// Workgroups are issued XCD-major: consecutive workgroup ids go round-robin
// over the 8 XCDs, so tile t runs on XCD t / (tiles / 8) and each XCD's L2
// sees the representatives of as few heads as possible; in the causal
// variant each XCD takes its tiles heaviest first.
#include <type_traits>

#include "bsa_device.hpp"
#include "bsa_launch.hpp"
#include "topk_list.hpp"

namespace bsa {
namespace {

constexpr int kTerms = 3;

// R tiles in flight ahead of the one computed in the hi-only pass.
constexpr int kSelectPrefetch = 1;

__device__ __forceinline__ int64_t xcd_tile(int causal) {
  const int64_t nwg = gridDim.x, bid = blockIdx.x;
  if (nwg % 8 != 0) return bid;
  const int64_t per = nwg / 8, local = bid / 8;
  return (bid % 8) * per + (causal ? per - 1 - local : local);
}

// The value lane l ^ 16 (row pair swap) or l ^ 32 (half swap) holds, with the
// gfx950 permlane swaps: called with the same register twice, the swap
// returns the partner's value in the second result for rows 0 and 2 (lower
// half) and in the first result for rows 1 and 3 (upper half).
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int lane) {
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}

// ------------------------------------------------------ score tiles ----
// A producer stages TB representatives in LDS and returns one lane's 4
// scores of a 16-block MFMA tile (tile): C[block 4g + j][query c16].

// LDS row pitch of the bf16 R tiles, in elements.  The A-operand read (16
// lanes, 16 rows, 16 bytes each) runs without bank conflicts at D + 16 (160 B
// rows for d = 64, 288 B for d = 128, measured on gfx950); at D + 8 half of
// the LDS cycles are conflicts.
template <int D>
constexpr int kRPitch = D + 16;

// One lane's 4 scores of MFMA tile mt from the 3-term R tile in LDS
// ([term][TB blocks][kRPitch] bf16) and its query's B operand.
template <int D, int TB, int NT = kTerms>
__device__ __forceinline__ f32x4 bf16_tile(const unsigned char* lds, const bf16x8 (&qb)[D / 32], int mt,
                                           int g, int c16) {
  constexpr int PITCH = kRPitch<D>;
  const __bf16* rs = reinterpret_cast<const __bf16*>(lds);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(rs + (t * TB + mt * 16 + c16) * PITCH + 8 * g + 32 * ks);
      acc = mfma_16x16x32_bf16(a, qb[ks], acc);
    }
  }
  return acc;
}

template <int D>
__device__ __forceinline__ void load_q_bf16(bf16x8 (&qb)[D / 32], const bf16_bits* __restrict__ q,
                                            int64_t qrow, int g) {
  const bf16_bits* qr = q + qrow * D + 8 * g;  // B operand: d = 8g + 32ks .. +7
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) qb[ks] = as_bf16x8(ld16(qr + 32 * ks));
}

// bf16 inputs, float32 representatives [block][d] split here into three bf16
// terms (the same split block_pool writes for the select kernel).  Panel
// kernel.
template <int D>
struct Bf16Tiles {
  using QT = bf16_bits;
  using Src = float;
  static constexpr int TB = 64;
  static constexpr int PITCH = kRPitch<D>;
  static constexpr int LDS_BYTES = kTerms * TB * PITCH * 2;
  bf16x8 qb[D / 32];

  __device__ __forceinline__ void load_q(const QT* __restrict__ q, int64_t qrow, int g) {
    load_q_bf16<D>(qb, q, qrow, g);
  }
  __device__ __forceinline__ static const Src* head_base(const Src* r, int64_t bh, int nb) {
    return r + bh * nb * D;
  }
  __device__ __forceinline__ static void stage(unsigned char* lds, const Src* __restrict__ rbase, int bt,
                                               int nb, int tid) {
    __bf16* rs = reinterpret_cast<__bf16*>(lds);
    for (int c = tid; c < TB * D / 4; c += 256) {
      const int r = c / (D / 4), col = (c % (D / 4)) * 4;
      const int beta = bt * TB + r;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (beta < nb) x = *reinterpret_cast<const float4*>(rbase + static_cast<int64_t>(beta) * D + col);
      float v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int t = 0; t < kTerms; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 h = f32_to_bf16(v[e]);
          rs[(t * TB + r) * PITCH + col + e] = h;
          v[e] -= static_cast<float>(h);
        }
      }
    }
  }
  template <int NT>
  __device__ __forceinline__ f32x4 tile(const unsigned char* lds, int mt, int g, int c16) const {
    return bf16_tile<D, TB>(lds, qb, mt, g, c16);
  }
};

// bf16 inputs, representatives pre-split by block_pool into term planes
// [term][beta][d] per head.  Select kernel: fetch() issues the global loads
// of a tile into registers, put() writes them to LDS, so the loads of tile
// bt + 1 are in flight while tile bt is computed.  Rows past the last block
// repeat the last block (their scores are never used).  NT = number of terms
// staged and multiplied: 3 (exact scores) or 1 (hi only, for the selection
// bound; put<1>() also tracks max |hi| per column for its error bound).
// QG query groups of 16 share each A-operand read from LDS: one read feeds
// QG MFMAs.  NTH = threads of the workgroup that stage the tile.
template <int D, int QG = 1, int NTH = 256, int TB_ = 32, int NTS = kTerms>
struct Bf16PlaneTiles {
  using QT = bf16_bits;
  using Src = bf16_bits;
  static constexpr int DIM = D;
  static constexpr int TB = TB_;                        // blocks per R tile
  static constexpr int PITCH = kRPitch<D>;
  // The hi-only tile type (NTS = 1) also reserves, after the plane, one
  // float per wave for set_norms' reduction.
  static constexpr bool kNorms = NTS == 1;
  static constexpr int NORM_OFF = NTS * TB * PITCH * 2;
  static constexpr int LDS_BYTES = NORM_OFF + (kNorms ? NTH / 16 : 0);  // NTS: terms staged at most
  static constexpr int CPR = D / 8;             // 16-byte chunks per block row
  static constexpr int PER = TB * CPR / NTH;    // chunks per thread and term
  static_assert(PER >= 1 && (TB * CPR) % NTH == 0, "whole chunks per thread");
  static_assert(NTH % CPR == 0, "a thread keeps one column chunk");
  static constexpr int PFD = kSelectPrefetch;  // R tiles in flight ahead of the one computed (hi-only walk)
  bf16x8 qb[QG][D / 32];
  uint4 pf[kTerms][PER];
  uint4 pf1[PFD > 1 ? PFD - 1 : 1][PER];  // further hi-only tiles in flight
  // c |q|_2 for each of this lane's queries, c = 2^-8 + 2^-13, and the
  // largest |hi|_2 of the head's blocks: qn * hmax bounds |exact score -
  // hi-only score| for every block (see set_norms).
  float qn[QG];
  float hmax = 0.f;

  // Query group gq of this lane: row qrow0 + 16 gq.
  __device__ __forceinline__ void load_q(const QT* __restrict__ q, int64_t qrow0, int g) {
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
      load_q_bf16<D>(qb[gq], q, qrow0 + 16 * gq, g);
      float ss = 0.f;  // this lane's D / 4 elements, then the query's 4 lanes
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = static_cast<float>(qb[gq][ks][e]);
          ss = __builtin_fmaf(x, x, ss);
        }
      qn[gq] = __builtin_sqrtf(sum_over_groups(ss)) * ((1.0f + 0x1.0p-16f) * (0x1.0p-8f + 0x1.0p-13f));
    }
  }
  // hmax = the largest hi-term norm |hi_beta|_2 of head bh's nb blocks
  // (each rounded up by block_pool), by the whole workgroup (NTH threads,
  // every one calling), through NTH / 64 floats of LDS at NORM_OFF.  For a
  // block, |exact score - hi-only score| <= sum_d |q_d| |r_d - hi_d| + the
  // fp32 rounding of both sums <= (2^-8 + 2^-13) |q|_2 |hi|_2 (hi is r
  // rounded to 8 significant bits, |r - hi| <= 2^-8 |hi|; Cauchy-Schwarz;
  // 2^-13 covers the roundings, and both norms are rounded up).  So the
  // largest hi-only score of a set of blocks, less qn * hmax, bounds from
  // below the largest exact score of the set: the block with the largest
  // hi-only score has an exact score at least that high.
  __device__ __forceinline__ void set_norms(const float* __restrict__ all, int64_t bh, int nb, unsigned char* lds) {
    const float* hn = all + bh * nb;
    float m = 0.f;
    for (int i = threadIdx.x; i < nb; i += NTH) m = fmaxf(m, hn[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float* red = reinterpret_cast<float*>(lds + NORM_OFF);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < NTH / 64; ++w) m = fmaxf(m, red[w]);
    hmax = m;
  }
  __device__ __forceinline__ static const Src* head_base(const Src* r, int64_t bh, int nb) {
    return r + bh * kTerms * nb * D;
  }
  // Loads of tile bt (all NT terms) into registers.  The hi-only walk keeps
  // PFD tiles in flight: fetch() then fills the last slot, and put() takes
  // the oldest and moves the others up.
  template <int NT>
  __device__ __forceinline__ void fetch(const Src* __restrict__ rbase, int nb, int bt, int tid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + NTH * u, r = c / CPR, col = (c % CPR) * 8;
      const int beta = min(bt * TB + r, nb - 1);
      if constexpr (NT == 1 && PFD > 1) {
        pf1[PFD - 2][u] = ld16(rbase + static_cast<uint32_t>(beta * D + col));
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          pf[t][u] = ld16(rbase + static_cast<uint32_t>((t * nb + beta) * D + col));
      }
    }
  }
  template <int NT>
  __device__ __forceinline__ void prime(const Src* __restrict__ rbase, int nb, int bt0, int tid) {
    fetch<NT>(rbase, nb, bt0, tid);
    if constexpr (NT == 1 && PFD > 1) {
#pragma unroll
      for (int u = 0; u < PER; ++u) pf[0][u] = pf1[PFD - 2][u];
#pragma unroll
      for (int i = 1; i < PFD; ++i) {
        fetch<NT>(rbase, nb, bt0 + i, tid);
#pragma unroll
        for (int u = 0; u < PER; ++u) pf1[i - 1][u] = pf1[PFD - 2][u];
      }
    }
  }
  template <int NT>
  __device__ __forceinline__ void put(unsigned char* lds, int tid) {
    __bf16* rs = reinterpret_cast<__bf16*>(lds);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + NTH * u, r = c / CPR, col = (c % CPR) * 8;
#pragma unroll
      for (int t = 0; t < NT; ++t) *reinterpret_cast<uint4*>(rs + (t * TB + r) * PITCH + col) = pf[t][u];
      if constexpr (NT == 1) {
        if constexpr (PFD > 1) {
          pf[0][u] = pf1[0][u];
#pragma unroll
          for (int i = 0; i + 1 < PFD - 1; ++i) pf1[i][u] = pf1[i + 1][u];
        }
      }
    }
  }
  // One lane's 4 scores of every MFMA tile of the R tile for each of its QG
  // query groups; the MT tiles' accumulation chains are interleaved (each
  // chain keeps the order of tiles(), so the scores are the same bits).
  template <int NT, int MT>
  __device__ __forceinline__ void tiles_all(const unsigned char* lds, int g, int c16, f32x4 (&acc)[MT][QG]) const {
    const __bf16* rs = reinterpret_cast<const __bf16*>(lds);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) acc[mt][gq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(rs + (t * TB + mt * 16 + c16) * PITCH + 8 * g + 32 * ks);
#pragma unroll
          for (int gq = 0; gq < QG; ++gq) acc[mt][gq] = mfma_16x16x32_bf16(a, qb[gq][ks], acc[mt][gq]);
        }
      }
    }
  }
  // One lane's 4 scores of MFMA tile mt for each of its QG query groups.
  template <int NT>
  __device__ __forceinline__ void tiles(const unsigned char* lds, int mt, int g, int c16, f32x4 (&acc)[QG]) const {
    const __bf16* rs = reinterpret_cast<const __bf16*>(lds);
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) acc[gq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(rs + (t * TB + mt * 16 + c16) * PITCH + 8 * g + 32 * ks);
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) acc[gq] = mfma_16x16x32_bf16(a, qb[gq][ks], acc[gq]);
      }
    }
  }
};

// fp32 inputs: v_mfma_f32_16x16x4_f32; slot (ks, g) carries d = KS*g + ks.
// stage() and tile() (one query group) for the panel kernel; fetch()/put()/
// tiles() as for Bf16PlaneTiles.
template <int D, int TB_, int QG = 1, int NTH = 256>
struct F32Tiles {
  using QT = float;
  using Src = float;
  static constexpr int DIM = D;
  static constexpr int TB = TB_;
  static constexpr int KS = D / 4;
  static constexpr int PITCH = D + 4;
  static constexpr int LDS_BYTES = TB * PITCH * 4;
  static constexpr int CPR = D / 4;             // 16-byte chunks per block row
  static constexpr int PER = TB * CPR / NTH;
  static_assert(PER >= 1 && (TB * CPR) % NTH == 0, "whole chunks per thread");
  float qf[QG][KS];
  float4 pf[PER];

  __device__ __forceinline__ void load_q(const QT* __restrict__ q, int64_t qrow0, int g) {
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
      const float* qr = q + (qrow0 + 16 * gq) * D + KS * g;
#pragma unroll
      for (int e = 0; e < KS; e += 4) {
        const float4 x = *reinterpret_cast<const float4*>(qr + e);
        qf[gq][e] = x.x; qf[gq][e + 1] = x.y; qf[gq][e + 2] = x.z; qf[gq][e + 3] = x.w;
      }
    }
  }
  __device__ __forceinline__ static const Src* head_base(const Src* r, int64_t bh, int nb) {
    return r + bh * nb * D;
  }
  __device__ __forceinline__ static void stage(unsigned char* lds, const Src* __restrict__ rbase, int bt,
                                               int nb, int tid) {
    float* rs = reinterpret_cast<float*>(lds);
    for (int c = tid; c < TB * D / 4; c += 256) {
      const int r = c / (D / 4), col = (c % (D / 4)) * 4;
      const int beta = bt * TB + r;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (beta < nb) x = *reinterpret_cast<const float4*>(rbase + static_cast<int64_t>(beta) * D + col);
      *reinterpret_cast<float4*>(rs + r * PITCH + col) = x;
    }
  }
  template <int NT>
  __device__ __forceinline__ void fetch(const Src* __restrict__ rbase, int nb, int bt, int tid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + NTH * u, r = c / CPR, col = (c % CPR) * 4;
      const int beta = min(bt * TB + r, nb - 1);
      pf[u] = *reinterpret_cast<const float4*>(rbase + static_cast<uint32_t>(beta * D + col));
    }
  }
  template <int NT>
  __device__ __forceinline__ void prime(const Src* __restrict__ rbase, int nb, int bt0, int tid) {
    fetch<NT>(rbase, nb, bt0, tid);
  }
  static constexpr int PFD = 1;
  template <int NT>
  __device__ __forceinline__ void put(unsigned char* lds, int tid) {
    float* rs = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + NTH * u, r = c / CPR, col = (c % CPR) * 4;
      *reinterpret_cast<float4*>(rs + r * PITCH + col) = pf[u];
    }
  }
  template <int NT>
  __device__ __forceinline__ f32x4 tile(const unsigned char* lds, int mt, int g, int c16) const {
    f32x4 acc[QG];
    tiles<NT>(lds, mt, g, c16, acc);
    return acc[0];
  }
  template <int NT>
  __device__ __forceinline__ void tiles(const unsigned char* lds, int mt, int g, int c16, f32x4 (&acc)[QG]) const {
    const float* rr = reinterpret_cast<const float*>(lds) + (mt * 16 + c16) * PITCH + KS * g;
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) acc[gq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float a = rr[ks];
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) acc[gq] = mfma_16x16x4_f32(a, qf[gq][ks], acc[gq]);
    }
  }
  template <int NT, int MT>
  __device__ __forceinline__ void tiles_all(const unsigned char* lds, int g, int c16, f32x4 (&acc)[MT][QG]) const {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) acc[mt][gq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float a = reinterpret_cast<const float*>(lds)[(mt * 16 + c16) * PITCH + KS * g + ks];
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) acc[mt][gq] = mfma_16x16x4_f32(a, qf[gq][ks], acc[mt][gq]);
      }
    }
  }
  // Pass 1 computes the same scores as pass 2 here: no error to bound.
  float qn[QG] = {};
  float hmax = 0.f;
  __device__ __forceinline__ void set_norms(const float*, int64_t, int, unsigned char*) {}
};

// Where a workgroup's 64 query rows sit, and which blocks they may select;
// nbt = number of TB-block tiles to walk.
struct TileInfo {
  int64_t tile_row, bh, qrow;
  int nb, nbt, nvalid, forced;
  int tid, lane, wave, g, c16;
  __device__ __forceinline__ TileInfo(int64_t row0, int n, int causal, int TB) {
    nb = n / kTile;
    tid = threadIdx.x;
    lane = tid & 63;
    wave = tid >> 6;
    g = lane >> 4;
    c16 = lane & 15;
    tile_row = row0 + xcd_tile(causal) * kTile;
    bh = tile_row / n;
    const int i0 = static_cast<int>(tile_row % n);
    qrow = tile_row + wave * 16 + c16;
    const int qblk = i0 / kTile;  // query block of all 64 rows
    nbt = causal ? qblk / TB + 1 : (nb + TB - 1) / TB;
    nvalid = causal ? qblk + 1 : nb;
    forced = causal ? qblk : -1;
  }
  // The score as the selection sees it: -inf for a block that is not a
  // candidate, +inf for the causal own block.
  __device__ __forceinline__ float cand(float s, int beta) const {
    const float x = beta == forced ? INFINITY : s;
    return beta < nvalid ? x : -INFINITY;
  }
};

// --------------------------------------------------------- panel mode ----
// panel rows: prows = rows of the chunk; panel[beta * prows + (qrow - row0)].
template <typename TL>
__global__ __launch_bounds__(256) void coarse_panel_kernel(const typename TL::QT* __restrict__ q,
                                                           const typename TL::Src* __restrict__ rsrc,
                                                           float* __restrict__ panel, int64_t row0,
                                                           int64_t prows, int n, int causal) {
  __shared__ __attribute__((aligned(16))) unsigned char rs[TL::LDS_BYTES];
  const TileInfo ti(row0, n, causal, TL::TB);
  TL sc;
  sc.load_q(q, ti.qrow, ti.g);
  const auto* rbase = TL::head_base(rsrc, ti.bh, ti.nb);
  const int64_t prow = ti.qrow - row0;
  for (int bt = 0; bt < ti.nbt; ++bt) {
    __syncthreads();
    TL::stage(rs, rbase, bt, ti.nb, ti.tid);
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < TL::TB / 16; ++mt) {
      if (bt * TL::TB + mt * 16 >= ti.nb) break;
      const f32x4 acc = sc.template tile<kTerms>(rs, mt, ti.g, ti.c16);
      const int beta0 = bt * TL::TB + mt * 16 + 4 * ti.g;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (beta0 + j < ti.nb) panel[static_cast<int64_t>(beta0 + j) * prows + prow] = acc[j];
    }
  }
}

// -------------------------------------------------------- select mode ----
// Is (va, ba) ranked above (vb, bb)?  Higher value first, then lower id.
__device__ __forceinline__ bool ranks_above(float va, int ba, float vb, int bb) {
  return va > vb || (va == vb && ba < bb);
}

// Compare-exchanges, descending.  Plain values: larger first.  (value,
// block) pairs: ranks_above order.
template <int N>
__device__ __forceinline__ void cx(float (&a)[N], int i, int j) {  // a[i] >= a[j] afterwards
  const float hi = fmaxf(a[i], a[j]), lo = fminf(a[i], a[j]);
  a[i] = hi;
  a[j] = lo;
}
template <int N>
__device__ __forceinline__ void cx(float (&v)[N], int (&b)[N], int i, int j) {
  const bool sw = ranks_above(v[j], b[j], v[i], b[i]);
  const float vi = v[i];
  const int bi = b[i];
  v[i] = sw ? v[j] : vi;
  b[i] = sw ? b[j] : bi;
  v[j] = sw ? vi : v[j];
  b[j] = sw ? bi : b[j];
}

// Bitonic sort of N values, descending.
template <int N>
__device__ __forceinline__ void sort_desc(float (&a)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          if ((i & size) == 0) cx(a, i, j);
          else cx(a, j, i);
        }
      }
    }
  }
}

// A bitonic sequence -> sorted descending.
template <int N>
__device__ __forceinline__ void bitonic_clean(float (&a)[N]) {
#pragma unroll
  for (int stride = N / 2; stride > 0; stride >>= 1)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((i ^ stride) > i) cx(a, i, i ^ stride);
}
template <int N>
__device__ __forceinline__ void bitonic_clean(float (&v)[N], int (&b)[N]) {
#pragma unroll
  for (int stride = N / 2; stride > 0; stride >>= 1)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((i ^ stride) > i) cx(v, b, i, i ^ stride);
}

// Both lanes of a pair (l, l ^ M) hold a sorted list; afterwards both hold
// the N largest of the two lists, sorted: c[i] = the larger of a[i] and the
// partner's a[N-1-i] is bitonic and holds the N largest.  Positions i and
// N-1-i are done together, before either is overwritten in both lanes, so no
// copy of the lists is needed.
template <int M, int N>
__device__ __forceinline__ void merge_top_unsorted(float (&a)[N], int lane) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float pi = __uint_as_float(lane_xor<M>(__float_as_uint(a[N - 1 - i]), lane));
    const float pj = __uint_as_float(lane_xor<M>(__float_as_uint(a[i]), lane));
    a[i] = fmaxf(a[i], pi);
    a[N - 1 - i] = fmaxf(a[N - 1 - i], pj);
  }
}
template <int M, int N>
__device__ __forceinline__ void merge_top(float (&a)[N], int lane) {
  merge_top_unsorted<M, N>(a, lane);
  bitonic_clean<N>(a);
}
template <int M, int N>
__device__ __forceinline__ void merge_top(float (&v)[N], int (&b)[N], int lane) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const int j = N - 1 - i;
    const float pvi = __uint_as_float(lane_xor<M>(__float_as_uint(v[j]), lane));
    const int pbi = static_cast<int>(lane_xor<M>(static_cast<uint32_t>(b[j]), lane));
    const float pvj = __uint_as_float(lane_xor<M>(__float_as_uint(v[i]), lane));
    const int pbj = static_cast<int>(lane_xor<M>(static_cast<uint32_t>(b[i]), lane));
    const bool ti = ranks_above(pvi, pbi, v[i], b[i]);
    const bool tj = ranks_above(pvj, pbj, v[j], b[j]);
    v[i] = ti ? pvi : v[i];
    b[i] = ti ? pbi : b[i];
    v[j] = tj ? pvj : v[j];
    b[j] = tj ? pbj : b[j];
  }
  bitonic_clean<N>(v, b);
}

// The t-th entry (t >= 1) of a descending array = the smallest of its first
// t entries; a reduction keeps the array in registers (a select chain on a
// dynamic index can be turned into a scratch-memory load).
template <int N>
__device__ __forceinline__ float kth_desc(const float (&a)[N], int t) {
  float r = a[0];
#pragma unroll
  for (int i = 1; i < N; ++i) r = fminf(r, i < t ? a[i] : INFINITY);
  return r;
}

// The keff-th largest of the values held by the 4 lanes g = 0..3 of one
// query (lanes c16 + 16 g), each sorted descending: after two pairwise
// merges every lane holds the N largest of the 4 N.  keff <= N, the same in
// every lane of the wave.  For keff = N the answer is the smallest of the N
// (the last merge is left unsorted); otherwise the list is sorted first.
template <int N>
__device__ __forceinline__ float kth_of_lanes(float (&a)[N], int keff, int lane) {
  merge_top<16, N>(a, lane);
  merge_top_unsorted<32, N>(a, lane);
  if (keff == N) {
    float r = a[0];
#pragma unroll
    for (int i = 1; i < N; ++i) r = fminf(r, a[i]);
    return r;
  }
  bitonic_clean<N>(a);
  return kth_desc<N>(a, keff);
}

// Write a query's selection in ascending block order: b[0 .. keff) are the
// selected blocks in any order (entries from keff on are ignored); lane g of
// the query's 4 writes entries g, g + 4, ... at their places, and -1 from keff
// up to topk.
template <int KL>
__device__ __forceinline__ void emit_selection(const int (&b)[KL], int g, int keff, int topk,
                                               int32_t* __restrict__ dst, int base) {
#pragma unroll
  for (int t0 = 0; t0 < KL; t0 += 4) {
    if (t0 + g < keff) {
      int me = b[t0];
#pragma unroll
      for (int e = 1; e < 4; ++e) me = g == e ? b[t0 + e] : me;
      int pos = 0;
#pragma unroll
      for (int u = 0; u < KL; ++u) pos += (u < keff && b[u] < me) ? 1 : 0;
      dst[pos] = me - base;
    }
  }
  for (int t = keff + g; t < topk; t += 4) dst[t] = -1;
}

// Sum over the query's 4 lanes.
__device__ __forceinline__ int sum4(int x, int lane) {
  x += static_cast<int>(lane_xor<16>(static_cast<uint32_t>(x), lane));
  return x + static_cast<int>(lane_xor<32>(static_cast<uint32_t>(x), lane));
}

// Ascending bitonic sort of the 4 E values held by the query's 4 lanes
// (lane g holds entries g E .. g E + E - 1): compare-exchanges at distances
// below E run inside the lane, the others between lanes g and g ^ (d / E)
// over the permlane swaps.  Afterwards lane g holds entries g E .. of the
// sorted order.
template <int E>
__device__ __forceinline__ void sort_asc_lanes(int (&b)[E], int g, int lane) {
  constexpr int N = 4 * E;
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1) {
      if (stride >= E) {
        const int m = stride / E;  // partner g ^ m: lane ^ 16 m
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const int o = static_cast<int>(m == 1 ? lane_xor<16>(static_cast<uint32_t>(b[i]), lane)
                                                : lane_xor<32>(static_cast<uint32_t>(b[i]), lane));
          const bool up = ((g * E + i) & size) == 0;
          const bool lower = (g & m) == 0;
          b[i] = up == lower ? min(b[i], o) : max(b[i], o);
        }
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const int j = i ^ stride;
          if (j > i) {
            const int lo = min(b[i], b[j]), hi = max(b[i], b[j]);
            const bool up = ((g * E + i) & size) == 0;
            b[i] = up ? lo : hi;
            b[j] = up ? hi : lo;
          }
        }
      }
    }
  }
}

// Where a select workgroup's queries sit: NW waves x QG query groups of 16
// rows; lane (g, c16) of wave w holds, for group gq, query row
// tile_row + 16 (w QG + gq) + c16.  All rows of a workgroup belong to one
// (batch, head), and (64-row query blocks being aligned to the 32-block R
// tiles) their query blocks lie in one R tile, the last one walked.
// With a block table (several sequences per head), the candidates start at
// the sequence's first block lo: the walk runs over tiles bt0 = lo / TB ..
// nbt - 1, and all rows of a workgroup (one 64-row query block) share lo.
template <int QG>
struct SelInfo {
  int64_t tile_row, bh, qrow0;
  int nb, nbt, bt0, lo;
  int nvalid[QG], forced[QG];
  int tid, lane, wave, g, c16;
  __device__ __forceinline__ SelInfo(int n, int causal, int TB, int NW, const int4* __restrict__ seqtab,
                                      int64_t tile) {
    const int rows = 16 * QG * NW;
    nb = n / kTile;
    tid = threadIdx.x;
    lane = tid & 63;
    wave = tid >> 6;
    g = lane >> 4;
    c16 = lane & 15;
    tile_row = tile * rows;
    bh = tile_row / n;
    const int i0 = static_cast<int>(tile_row % n);
    qrow0 = tile_row + 16 * QG * wave + c16;
    int hi = nb;
    lo = 0;
    if (seqtab) {
      const int4 e = seqtab[i0 / kTile];
      lo = e.x;
      hi = e.y;
    }
    const int qlast = (i0 + rows - 1) / kTile;  // query block of the workgroup's last row
    nbt = causal ? qlast / TB + 1 : (hi + TB - 1) / TB;
    bt0 = lo / TB;
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
      const int qblk = (i0 + 16 * (QG * wave + gq)) / kTile;
      nvalid[gq] = causal ? qblk + 1 : hi;
      forced[gq] = causal ? qblk : -1;
    }
  }
  // The score as the selection sees it: -inf for a block that is not a
  // candidate, +inf for the causal own block.
  __device__ __forceinline__ float cand(int gq, float s, int beta) const {
    const float x = beta == forced[gq] ? INFINITY : s;
    return (beta < nvalid[gq] && beta >= lo) ? x : -INFINITY;
  }
};

// Stream the tiles of the workgroup's representatives through LDS, register-
// prefetching tile bt + 1 while tile bt is computed, and hand each 16-block
// MFMA tile (its QG accumulators) to fast(h, mt, b0, acc) or slow(...) (b0 =
// first block of the MFMA tile, h = bt mod NH as a compile-time value: the
// loop is unrolled by NH).  Every block of a tile before the last is an
// ordinary candidate for every query group (below each group's own block),
// so only the last tile takes the checked slow().
template <int NH, int NT, int QG, int NTH, typename TL, typename FF, typename FS>
__device__ __forceinline__ void walk(TL& sc, unsigned char* rs, const typename TL::Src* rbase,
                                     const SelInfo<QG>& ti, FF&& fast, FS&& slow) {
  constexpr int MT = TL::TB / 16;
  constexpr int PF = NT == 1 ? TL::PFD : 1;  // tiles loaded ahead
  sc.template prime<NT>(rbase, ti.nb, ti.bt0, ti.tid);
  f32x4 acc[MT][QG];
  int bt0 = ti.bt0;
  // A first tile that starts before the sequence's first block (and is not
  // the last) is checked too.
  if (ti.lo % TL::TB != 0 && bt0 + 1 < ti.nbt) {
    __syncthreads();
    sc.template put<NT>(rs, ti.tid);
    sc.template fetch<NT>(rbase, ti.nb, bt0 + PF, ti.tid);
    __syncthreads();
    sc.template tiles_all<NT, MT>(rs, ti.g, ti.c16, acc);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) slow(0, mt, bt0 * TL::TB + mt * 16, acc[mt]);
    ++bt0;
  }
  // Steady state: NH tiles per iteration, none of them the last, so the body
  // has no branches and the slot index h stays a compile-time value.
  for (; bt0 + NH < ti.nbt; bt0 += NH) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int bt = bt0 + h;
      __syncthreads();
      sc.template put<NT>(rs, ti.tid);
      sc.template fetch<NT>(rbase, ti.nb, bt + PF, ti.tid);
      __syncthreads();
      sc.template tiles_all<NT, MT>(rs, ti.g, ti.c16, acc);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) fast(h, mt, bt * TL::TB + mt * 16, acc[mt]);
    }
  }
  // The remaining 1 .. NH tiles; the last one takes the checked slow().
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int bt = bt0 + h;
    if (bt < ti.nbt) {
      __syncthreads();
      sc.template put<NT>(rs, ti.tid);
      const bool last = bt + 1 == ti.nbt;
      if (bt + PF < ti.nbt) sc.template fetch<NT>(rbase, ti.nb, bt + PF, ti.tid);
      __syncthreads();
      sc.template tiles_all<NT, MT>(rs, ti.g, ti.c16, acc);
      if (!last) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) fast(h, mt, bt * TL::TB + mt * 16, acc[mt]);
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int b0 = bt * TL::TB + mt * 16;
          if (b0 >= ti.nb) break;
          slow(h, mt, b0, acc[mt]);
        }
      }
    }
  }
}

// Exact selection of a workgroup's queries: every score offered to exact
// register top-KL lists (topk_list.hpp), merged over the query's 4 lanes and
// written in ascending block order.  The slow path behind the candidate
// slots, taken only when they overflow twice.
template <typename TL, int KL, int QG, int NTH>
__device__ __forceinline__ void exact_select(TL& sc, unsigned char* rs, const typename TL::Src* rbase,
                                             const SelInfo<QG>& ti, const int (&keff)[QG], int topk,
                                             int32_t* __restrict__ idx) {
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    TopList<KL> l;
    l.init();
    walk<1, kTerms, QG, NTH>(sc, rs, rbase, ti,
         [&](int, int, int b0, const f32x4 (&acc)[QG]) {
           f32x4 v = acc[0];
#pragma unroll
           for (int e = 1; e < QG; ++e) v = gq == e ? acc[e] : v;
#pragma unroll
           for (int j = 0; j < 4; ++j) l.offer(v[j], b0 + 4 * ti.g + j);
         },
         [&](int, int, int b0, const f32x4 (&acc)[QG]) {
           f32x4 v = acc[0];
#pragma unroll
           for (int e = 1; e < QG; ++e) v = gq == e ? acc[e] : v;
#pragma unroll
           for (int j = 0; j < 4; ++j) l.offer(ti.cand(gq, v[j], b0 + 4 * ti.g + j), b0 + 4 * ti.g + j);
         });
    merge_top<16, KL>(l.v, l.b, ti.lane);
    merge_top<32, KL>(l.v, l.b, ti.lane);
    emit_selection<KL>(l.b, ti.g, keff[gq], topk, idx + (ti.qrow0 + 16 * gq) * topk, ti.lo);
  }
}

// MINW: waves per SIMD the register budget is sized for.  NW waves per
// workgroup, QG query groups of 16 per wave.
// The tile type of the hi-only first pass: bf16 planes take R tiles of twice
// the three-term tiles' blocks there (one staged term fits the LDS those
// use; at 64 blocks each tile gives four independent MFMA chains); fp32 keeps
// its tiles.
template <typename TL>
struct Pass1Tiles {
  using type = TL;
};
template <int D, int QG, int NTH, int TB_, int NTS>
struct Pass1Tiles<Bf16PlaneTiles<D, QG, NTH, TB_, NTS>> {
  using type = Bf16PlaneTiles<D, QG, NTH, 2 * TB_, 1>;
};

template <typename TL, int KL, int GM, int CAP, int MINW, int QG, int NW, bool SPLIT>
__global__ __launch_bounds__(64 * NW, MINW) void coarse_select_kernel(const typename TL::QT* __restrict__ q,
                                                                      const typename TL::Src* __restrict__ rsrc,
                                                                      int32_t* __restrict__ idx, int n,
                                                                      int topk, const HeadBudget budget,
                                                                      int causal,
                                                                      const int4* __restrict__ seqtab,
                                                                      const float* __restrict__ hinorm,
                                                                      int32_t* __restrict__ fallbacks,
                                                                      int32_t* __restrict__ repair_count,
                                                                      int32_t* __restrict__ repair_clear,
                                                                      int32_t* __restrict__ repair_list,
                                                                      const typename TL::QT* __restrict__ warm) {
  using TL1 = typename Pass1Tiles<TL>::type;
  // split instance: this call lists its exact redos at repair_count, and
  // clears the other counter for the next call (no kernel of this call uses
  // it)
  if (SPLIT && blockIdx.x == 0 && threadIdx.x == 0) *repair_clear = 0;
  constexpr int NTH = 64 * NW;
  constexpr int MT = TL1::TB / 16;    // MFMA tiles per R tile of pass 1
  constexpr int NS = 16 * GM;         // group slots per lane
  constexpr int NH = NS / (4 * MT) > 0 ? NS / (4 * MT) : 1;  // R tiles per cycle of slots
  static_assert(NS % (4 * MT) == 0, "a cycle of slots covers whole R tiles");
  constexpr int ROWS = 16 * QG * NW;  // queries per workgroup
  // The R tile buffer (the hi-only tiles with set_norms' reduction slots, or
  // the three-term tiles) also holds, at the end, the selection lists (a row of 33 per
  // query) and a slot per lane.
  constexpr int LIST_BYTES = (ROWS * 33 + NTH) * 4;
  constexpr int RS_T = TL::LDS_BYTES > TL1::LDS_BYTES ? TL::LDS_BYTES : TL1::LDS_BYTES;
  constexpr int RS_BYTES = RS_T > LIST_BYTES ? RS_T : LIST_BYTES;
  static_assert(CAP <= KL && KL <= 32, "candidate slots are tracked in a 32-bit mask");
  __shared__ __attribute__((aligned(16))) unsigned char rs[RS_BYTES];
  // per lane and query group: candidate scores and blocks
  __shared__ float cv[NW][QG][CAP][64];
  __shared__ uint16_t cb[NW][QG][CAP][64];
  static_assert(ROWS == kTile, "a workgroup's rows are one query block, so one sequence");
  const int64_t tile = xcd_tile(causal);
  const SelInfo<QG> ti(n, causal, TL::TB, NW, seqtab, tile);
  const SelInfo<QG> ti1(n, causal, TL1::TB, NW, seqtab, tile);  // the same rows, walked in pass-1 tiles
  const auto* rbase = TL::head_base(rsrc, ti.bh, ti.nb);
  const int kh = budget.k[ti.bh % budget.heads];  // this head's budget (<= topk <= KL)
  int keff[QG];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) keff[gq] = kh < ti.nvalid[gq] - ti.lo ? kh : ti.nvalid[gq] - ti.lo;

  // pass 1: group maxima.  The lane's block 16 (MT bt + mt) + 4 g + j goes to
  // slot 4 ((MT bt + mt) mod 4 GM) + j: G = 64 GM groups over the 4 lanes.
  float a[QG][NS];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq)
#pragma unroll
    for (int u = 0; u < NS; ++u) a[gq][u] = -INFINITY;
  // Pass 1 may run on approximate scores (bf16: the hi term alone): each
  // group's maximum enters less the error bound of the head's blocks
  // (set_norms), a lower bound of the group's largest exact score, so tau
  // stays a bound for the exact scores.
  float tau[QG];
  // The V rows of the workgroup's queries (warm, when given), read and
  // discarded so the attention kernel finds V in the Infinity Cache.  Issued
  // before the query rows and used (XOR, an empty asm) after them, they add
  // no wait of their own.
  constexpr int VCH = kTile * TL::DIM * static_cast<int>(sizeof(typename TL::QT)) / 16;
  constexpr int VPT = (VCH + NTH - 1) / NTH;
  uint4 vw[VPT];
  if (warm) {
    const uint4* vsrc = reinterpret_cast<const uint4*>(warm + ti.tile_row * TL::DIM);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + NTH * i;
      vw[i] = c < VCH ? vsrc[c] : make_uint4(0, 0, 0, 0);
    }
  }
  {
    TL1 sc1;
    sc1.set_norms(hinorm, ti.bh, ti.nb, rs);
    sc1.load_q(q, ti.qrow0, ti.g);
    if (warm) {
      uint32_t seen = 0;
#pragma unroll
      for (int i = 0; i < VPT; ++i) seen ^= vw[i].x ^ vw[i].y ^ vw[i].z ^ vw[i].w;
      asm volatile("" ::"v"(seen));
    }
    auto group_max = [&](bool checked, int h, int mt, int b0, const f32x4 (&acc)[QG]) {
#pragma unroll
      for (int gq = 0; gq < QG; ++gq)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = checked ? ti.cand(gq, acc[gq][j], b0 + 4 * ti.g + j) : acc[gq][j];
          a[gq][4 * (MT * h + mt) + j] = fmaxf(a[gq][4 * (MT * h + mt) + j], x);
        }
    };
    walk<NH, 1, QG, NTH>(sc1, rs, rbase, ti1,
                         [&](int h, int mt, int b0, const f32x4 (&acc)[QG]) { group_max(false, h, mt, b0, acc); },
                         [&](int h, int mt, int b0, const f32x4 (&acc)[QG]) { group_max(true, h, mt, b0, acc); });
    // the groups' maxima, less the bound (infinite maxima stay infinite)
#pragma unroll
    for (int gq = 0; gq < QG; ++gq)
#pragma unroll
      for (int u = 0; u < NS; ++u) a[gq][u] = __builtin_fmaf(-sc1.qn[gq], sc1.hmax, a[gq][u]);
  }
  TL sc;
  sc.load_q(q, ti.qrow0, ti.g);
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    sort_desc<NS>(a[gq]);
    tau[gq] = kth_of_lanes<NS>(a[gq], keff[gq], ti.lane);
  }

  // pass 2: the candidates >= tau, in ascending block order
  int cnt[QG];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) cnt[gq] = 0;
  auto append = [&](bool checked, int b0, const f32x4 (&acc)[QG]) {
#pragma unroll
    for (int gq = 0; gq < QG; ++gq)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int beta = b0 + 4 * ti.g + j;
        const float x = checked ? ti.cand(gq, acc[gq][j], beta) : acc[gq][j];
        // past CAP candidates the lane overwrites its last slot: the count
        // still grows, and a count above CAP sends the workgroup to the
        // exact redo below
        const int slot = cnt[gq] < CAP ? cnt[gq] : CAP - 1;
        if (x >= tau[gq]) {
          cv[ti.wave][gq][slot][ti.lane] = x;
          cb[ti.wave][gq][slot][ti.lane] = static_cast<uint16_t>(beta);
          ++cnt[gq];
        }
      }
  };
  // A workgroup in which some lane's candidates overflowed its slots walks a
  // second time with a higher bound: tau2 = the k_eff-th largest of the
  // candidates its lanes did keep (real scores, so at least k_eff scores are
  // >= tau2, and every score of the answer is).  Only if that also overflows
  // does it take the exact redo below.
  walk<1, kTerms, QG, NTH>(sc, rs, rbase, ti,
                           [&](int, int, int b0, const f32x4 (&acc)[QG]) { append(false, b0, acc); },
                           [&](int, int, int b0, const f32x4 (&acc)[QG]) { append(true, b0, acc); });
  bool bad = false;
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) bad = bad || cnt[gq] > CAP || sum4(cnt[gq], ti.lane) < keff[gq];
  int redo = __syncthreads_or(bad);
  if (redo) {  // rare: its own copy of the walk keeps the common path's code as it was
    if (fallbacks && threadIdx.x == 0) atomicAdd(fallbacks, 1);
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
      float c[KL];
#pragma unroll
      for (int i = 0; i < KL; ++i) c[i] = (i < CAP && i < cnt[gq]) ? cv[ti.wave][gq][i < CAP ? i : 0][ti.lane] : -INFINITY;
      sort_desc<KL>(c);
      tau[gq] = fmaxf(tau[gq], kth_of_lanes<KL>(c, keff[gq], ti.lane));
      cnt[gq] = 0;
    }
    walk<1, kTerms, QG, NTH>(sc, rs, rbase, ti,
                             [&](int, int, int b0, const f32x4 (&acc)[QG]) { append(false, b0, acc); },
                             [&](int, int, int b0, const f32x4 (&acc)[QG]) { append(true, b0, acc); });
    bad = false;
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) bad = bad || cnt[gq] > CAP || sum4(cnt[gq], ti.lane) < keff[gq];
    redo = __syncthreads_or(bad);
  }

  if (!redo) {
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
      int32_t* dst = idx + (ti.qrow0 + 16 * gq) * topk;
      const int kq = keff[gq];
      // The lane's candidate scores, read once into registers (-inf past cnt
      // and past the CAP stored slots, up to the list length KL), in ascending
      // block order.
      const float(&lv)[CAP][64] = cv[ti.wave][gq];
      const uint16_t(&lb)[CAP][64] = cb[ti.wave][gq];
      float x[KL];
#pragma unroll
      for (int i = 0; i < KL; ++i) x[i] = (i < CAP && i < cnt[gq]) ? lv[i < CAP ? i : 0][ti.lane] : -INFINITY;
      // T = the keff-th largest candidate score of the query: every lane sorts
      // a copy of its scores, two pairwise merges give all 4 lanes the query's
      // top CAP.
      float c[KL];
#pragma unroll
      for (int i = 0; i < KL; ++i) c[i] = x[i];
      sort_desc<KL>(c);
      const float T = kth_of_lanes<KL>(c, kq, ti.lane);
      // Selected: scores above T, and the lowest-block `need` of those equal
      // to T; when exactly `need` candidates equal T (the usual case) all are.
      uint32_t gtb = 0u, eqb = 0u;
#pragma unroll
      for (int i = 0; i < CAP; ++i) {
        gtb |= x[i] > T ? (1u << i) : 0u;
        eqb |= x[i] == T ? (1u << i) : 0u;
      }
      const int need = kq - sum4(__popc(gtb), ti.lane);
      const bool all_ties = sum4(__popc(eqb), ti.lane) == need;
      uint32_t selbits = gtb | (all_ties ? eqb : 0u);
      const int cn = cnt[gq];
      const int cnt16 = static_cast<int>(lane_xor<16>(static_cast<uint32_t>(cn), ti.lane));
      const int cnt32 = static_cast<int>(lane_xor<32>(static_cast<uint32_t>(cn), ti.lane));
      const int cnt48 = static_cast<int>(lane_xor<32>(static_cast<uint32_t>(cnt16), ti.lane));
      if (!all_ties) {
        // A tie's rank among the query's ties = ties before it in its own lane
        // (ascending blocks) + ties with lower blocks in the other 3 lanes.
        int ties_before = 0;
#pragma unroll
        for (int i = 0; i < CAP; ++i) {
          if (x[i] == T) {
            int r = ties_before++;
            for (int m = 1; m < 4; ++m) {
              const int ln = ti.lane ^ (16 * m);
              const int cm = m == 1 ? cnt16 : m == 2 ? cnt32 : cnt48;
              for (int jj = 0; jj < cm; ++jj) r += (lv[jj][ln] == T && lb[jj][ln] < lb[i][ti.lane]) ? 1 : 0;
            }
            selbits |= r < need ? (1u << i) : 0u;
          }
        }
      }
      // The query's selection into its row of an LDS list (the R tile buffer
      // is free now), this lane's part after those of lanes g' < g; a lane
      // writes unselected entries to a slot of its own.
      const int ns = __popc(selbits);
      const int n16 = static_cast<int>(lane_xor<16>(static_cast<uint32_t>(ns), ti.lane));
      const int n32 = static_cast<int>(lane_xor<32>(static_cast<uint32_t>(ns), ti.lane));
      const int n48 = static_cast<int>(lane_xor<32>(static_cast<uint32_t>(n16), ti.lane));
      int p = ((ti.g & 1) ? n16 : 0) + ((ti.g & 2) ? n32 + n48 : 0);
      const int qslot = 16 * (QG * ti.wave + gq) + ti.c16;
      int* list = reinterpret_cast<int*>(rs) + qslot * 33;  // odd pitch: no bank conflicts
      int* own = reinterpret_cast<int*>(rs) + ROWS * 33 + ti.tid;
#pragma unroll
      for (int i = 0; i < CAP; ++i) {
        const bool sel = (selbits >> i) & 1u;
        *(sel ? list + p : own) = lb[i][ti.lane];
        p += sel ? 1 : 0;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      // The query's 4 lanes sort its keff blocks together, lane g taking
      // entries g E .. g E + E - 1 of the row (E = KL / 4; padding past keff
      // sorts last and becomes -1), and store them: whole 16-byte chunks
      // when the row allows, else entry by entry.
      constexpr int E = KL / 4;
      int b[E];
#pragma unroll
      for (int i = 0; i < E; ++i) b[i] = ti.g * E + i < kq ? list[ti.g * E + i] : 0x7fffffff;
      sort_asc_lanes<E>(b, ti.g, ti.lane);
#pragma unroll
      for (int i = 0; i < E; ++i) b[i] = ti.g * E + i < kq ? b[i] - ti.lo : -1;
      if (E % 4 == 0 && ((reinterpret_cast<uintptr_t>(dst) | static_cast<uintptr_t>(topk) * 4u) & 15u) == 0) {
#pragma unroll
        for (int c0 = 0; c0 < E; c0 += 4) {
          const int t = ti.g * E + c0;
          if (t < topk) *reinterpret_cast<int4*>(dst + t) = make_int4(b[c0], b[c0 + 1], b[c0 + 2], b[c0 + 3]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const int t = ti.g * E + i;
          if (t < topk) dst[t] = b[i];
        }
      }
    }
  } else {
    // slots overflowed again somewhere in the workgroup: the exact walk,
    // here or, for the split instance, in the repair kernel (counted when
    // asked, one vector atomic per such workgroup)
    if constexpr (SPLIT) {
      if (threadIdx.x == 0) {
        const int32_t i = atomicAdd(repair_count, 1);
        if (i < static_cast<int32_t>(gridDim.x)) repair_list[i] = static_cast<int32_t>(tile);
      }
    } else {
      if (fallbacks && threadIdx.x == 0) atomicAdd(fallbacks + 1, 1);
      exact_select<TL, KL, QG, NTH>(sc, rs, rbase, ti, keff, topk, idx);
    }
  }
}

// The exact redo of a workgroup's selection for a tile listed by the split
// instance of the select kernel (bf16, d = 128, k > 16): without the
// register lists of the exact walk the select kernel fits in 152 VGPRs, so 3
// workgroups per CU run it without spilling.  count[0] tiles are listed
// (any tile number outside this call's tiles is skipped); a grid-stride loop
// over them, every workgroup leaving when the list is done.
template <typename TL, int KL, int QG, int NW>
__global__ __launch_bounds__(64 * NW) void coarse_repair_kernel(const typename TL::QT* __restrict__ q,
                                                                const typename TL::Src* __restrict__ rsrc,
                                                                int32_t* __restrict__ idx, int n, int topk,
                                                                const HeadBudget budget, int causal,
                                                                const int4* __restrict__ seqtab,
                                                                const int32_t* __restrict__ repair_count,
                                                                const int32_t* __restrict__ repair_list,
                                                                int32_t ntiles, int32_t* __restrict__ fallbacks) {
  constexpr int NTH = 64 * NW;
  __shared__ __attribute__((aligned(16))) unsigned char rs[TL::LDS_BYTES];
  const int32_t listed = *repair_count;
  const int32_t total = listed < ntiles ? listed : ntiles;
  for (int32_t i = blockIdx.x; i < total; i += gridDim.x) {
    const int32_t tile = repair_list[i];
    if (tile < 0 || tile >= ntiles) continue;  // workgroup-uniform
    const SelInfo<QG> ti(n, causal, TL::TB, NW, seqtab, tile);
    const auto* rbase = TL::head_base(rsrc, ti.bh, ti.nb);
    const int kh = budget.k[ti.bh % budget.heads];
    int keff[QG];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) keff[gq] = kh < ti.nvalid[gq] - ti.lo ? kh : ti.nvalid[gq] - ti.lo;
    TL sc;
    sc.load_q(q, ti.qrow0, ti.g);
    if (fallbacks && threadIdx.x == 0) atomicAdd(fallbacks + 1, 1);
    exact_select<TL, KL, QG, NTH>(sc, rs, rbase, ti, keff, topk, idx);
  }
}

// ------------------------------------------------------------ launch ----
template <typename TL>
void launch_panel(const void* q, const void* rsrc, float* panel, int64_t row0, int64_t rows, int n,
                  int causal, hipStream_t s) {
  hipLaunchKernelGGL((coarse_panel_kernel<TL>), dim3(static_cast<unsigned>(rows / kTile)), dim3(256), 0, s,
                     static_cast<const typename TL::QT*>(q), static_cast<const typename TL::Src*>(rsrc),
                     panel, row0, rows, n, causal);
}

// Per-call extras of the select launch: the repair state of the split
// instance (two counters, one per call parity, and a list of one entry per
// select workgroup), the blocks' hi-term norms (bf16, after the split
// planes) and the V to read ahead (or null).
struct Repair {
  int32_t* counters = nullptr;
  int32_t* list = nullptr;
  int parity = 0;
  const float* hinorm = nullptr;
  const void* warm = nullptr;
};

template <typename TL, int KL, int GM, int CAP, int MINW, int QG, int NW, bool SPLIT = false>
void launch_select(const void* q, const void* rsrc, int32_t* idx, int64_t rows, int n, int topk,
                   const HeadBudget& hb, int causal, const int4* seqtab, int32_t* fallbacks, const Repair& rp,
                   hipStream_t s) {
  constexpr int ROWS = 16 * QG * NW;
  const int64_t tiles = rows / ROWS;
  int32_t* count = SPLIT ? rp.counters + rp.parity : nullptr;
  int32_t* clear = SPLIT ? rp.counters + (1 - rp.parity) : nullptr;
  hipLaunchKernelGGL((coarse_select_kernel<TL, KL, GM, CAP, MINW, QG, NW, SPLIT>), dim3(static_cast<unsigned>(tiles)),
                     dim3(64 * NW), 0, s, static_cast<const typename TL::QT*>(q),
                     static_cast<const typename TL::Src*>(rsrc), idx, n, topk, hb, causal, seqtab, rp.hinorm, fallbacks,
                     count, clear, SPLIT ? rp.list : nullptr, static_cast<const typename TL::QT*>(rp.warm));
  if constexpr (SPLIT) {
    const int64_t grid = tiles < 1024 ? tiles : 1024;
    hipLaunchKernelGGL((coarse_repair_kernel<TL, KL, QG, NW>), dim3(static_cast<unsigned>(grid)), dim3(64 * NW), 0, s,
                       static_cast<const typename TL::QT*>(q), static_cast<const typename TL::Src*>(rsrc), idx, n,
                       topk, hb, causal, seqtab, count, rp.list, static_cast<int32_t>(tiles), fallbacks);
  }
}

// One 16-query group per wave, four waves per workgroup; the register budget
// allows 4 waves per SIMD for bf16 d = 64 and k <= 16, else 3 (2 for k > 16,
// whose candidate lists are twice as long).  bf16 at d = 128 and k > 16 (the
// long causal workload) runs 3 workgroups per CU instead of 2: 24 candidate
// slots per lane (lists still sorted 32 long; a lane with more candidates
// takes the second walk, 3.5 % of its workgroups), three-term R tiles of 16
// blocks and hi-only tiles of 32, 51 KB of LDS (selection 2.00 -> 1.82 ms).
template <template <int, int, int> class TLT, int D>
void launch_select_k(const void* q, const void* rsrc, int32_t* idx, int64_t rows, int n, int topk,
                     const HeadBudget& hb, int causal, const int4* seqtab, int32_t* fb, const Repair& rp,
                     hipStream_t s) {
  constexpr int M1 = (D == 64 && std::is_same<typename TLT<D, 1, 256>::QT, bf16_bits>::value) ? 4 : 3;
  if (topk <= 8) launch_select<TLT<D, 1, 256>, 8, 1, 8, M1, 1, 4>(q, rsrc, idx, rows, n, topk, hb, causal, seqtab, fb, rp, s);
  else if (topk <= 16) launch_select<TLT<D, 1, 256>, 16, 1, 16, M1, 1, 4>(q, rsrc, idx, rows, n, topk, hb, causal, seqtab, fb, rp, s);
  else if constexpr (D == 128 && std::is_same<typename TLT<D, 1, 256>::QT, bf16_bits>::value)
    launch_select<Bf16PlaneTiles<D, 1, 256, 16, kTerms>, 32, 2, 24, 3, 1, 4, true>(q, rsrc, idx, rows, n, topk, hb,
                                                                                  causal, seqtab, fb, rp, s);
  else launch_select<TLT<D, 1, 256>, 32, 2, 32, 2, 1, 4>(q, rsrc, idx, rows, n, topk, hb, causal, seqtab, fb, rp, s);
}

template <int D, int QG, int NTH>
using PlaneT = Bf16PlaneTiles<D, QG, NTH>;
template <int D, int QG, int NTH>
using F32T = F32Tiles<D, 32, QG, NTH>;

}  // namespace

hipError_t launch_coarse_score(const void* q, const float* repr, float* panel, int64_t row0,
                               int64_t rows, int n, int d, bsa_dtype dtype, int causal,
                               hipStream_t stream) {
  if (dtype == BSA_BF16) {
    if (d == 64) launch_panel<Bf16Tiles<64>>(q, repr, panel, row0, rows, n, causal, stream);
    else launch_panel<Bf16Tiles<128>>(q, repr, panel, row0, rows, n, causal, stream);
  } else {
    if (d == 64) launch_panel<F32Tiles<64, 64>>(q, repr, panel, row0, rows, n, causal, stream);
    else launch_panel<F32Tiles<128, 64>>(q, repr, panel, row0, rows, n, causal, stream);
  }
  return hipGetLastError();
}

hipError_t launch_coarse_select(const void* q, const float* repr, const uint16_t* repr_split,
                                int32_t* idx, int64_t rows, int n, int d, bsa_dtype dtype,
                                int topk, const HeadBudget& hb, int causal, hipStream_t stream,
                                const int4* seqtab, int32_t* fallbacks, int32_t* repair_counters,
                                int32_t* repair_list, int repair_parity, const void* warm) {
  Repair rp;
  rp.counters = repair_counters;
  rp.list = repair_list;
  rp.parity = repair_parity;
  if (rows * d * (dtype == BSA_BF16 ? 2 : 4) <= kWarmMaxBytes) rp.warm = warm;
  if (dtype == BSA_BF16) rp.hinorm = split_norms(const_cast<uint16_t*>(repr_split), rows / n, n / kTile, d);
  if (select_uses_repair(d, dtype, topk) && (!repair_counters || !repair_list)) return hipErrorInvalidValue;
  if (dtype == BSA_BF16) {
    if (d == 64) launch_select_k<PlaneT, 64>(q, repr_split, idx, rows, n, topk, hb, causal, seqtab, fallbacks, rp, stream);
    else launch_select_k<PlaneT, 128>(q, repr_split, idx, rows, n, topk, hb, causal, seqtab, fallbacks, rp, stream);
  } else {
    if (d == 64) launch_select_k<F32T, 64>(q, repr, idx, rows, n, topk, hb, causal, seqtab, fallbacks, rp, stream);
    else launch_select_k<F32T, 128>(q, repr, idx, rows, n, topk, hb, causal, seqtab, fallbacks, rp, stream);
  }
  return hipGetLastError();
}

}  // namespace bsa
