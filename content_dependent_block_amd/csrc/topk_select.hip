// topk_select.hip -- Stage 1 selection: each query keeps its k highest-scoring
// blocks (nishantmodi.me "sparse-attention-triton-bench", section "Stage 2:
// fine attention": take the top-k highest-scoring blocks per query; the
// indices are int32, section "Two things I wish I knew").
//
// Semantics: candidates are all n/64 blocks, or in the causal variant the
// blocks up to the query's own block, which is always kept.  k_eff =
// min(k, #candidates).  Equal scores go to the lower block index and -0 equals
// +0.  Output: the k_eff indices in ascending order, then -1 up to k.
//
// One wavefront per query row; lane l holds the scores of blocks l + 64*j.
// Scores become order-preserving uint32 keys (-0 folded onto +0; the forced
// own block gets 0xFFFFFFFF, above every float; non-candidates get 0, below
// every float).  A binary radix search over the 32 key bits finds the k_eff-th
// largest key T with one ballot + popcount per bit and per register; it stops
// early as soon as exactly k_eff keys are >= the current prefix.  The keys
// above T, plus the lowest-indexed keys equal to T, are then written in
// ascending index order with ballot / mbcnt prefix counts, so no sort is
// needed.  All control flow is wave-uniform.
#include "bsa_device.hpp"
#include "bsa_launch.hpp"

namespace bsa {
namespace {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int NPER>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ panel,
                                                   int32_t* __restrict__ idx, int64_t row0,
                                                   int64_t rows, int n, int topk, int causal) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int nb = n / kTile;
  const int64_t grow = row0 + r;
  const int qb = static_cast<int>(grow % n) / kTile;
  const int nvalid = causal ? (qb + 1 < nb ? qb + 1 : nb) : nb;
  const int keff = topk < nvalid ? topk : nvalid;
  const float* src = panel + r * nb;

  uint32_t key[NPER];
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const int e = lane + 64 * j;
    uint32_t kk = 0u;
    if (e < nvalid) kk = (causal && e == qb) ? 0xFFFFFFFFu : order_key(src[e]);
    key[j] = kk;
  }

  // Radix search for the threshold.
  uint32_t prefix = 0u, thr = 0u;
  bool exact = false;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = prefix | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NPER; ++j) cnt += __popcll(ballot(key[j] >= cand));
    if (cnt >= keff) {
      prefix = cand;
      if (cnt == keff) {
        thr = cand - 1u;  // exactly keff keys are > thr
        exact = true;
        break;
      }
    }
  }
  if (!exact) thr = prefix;  // the keff-th largest key
  int gt = 0;
#pragma unroll
  for (int j = 0; j < NPER; ++j) gt += __popcll(ballot(key[j] > thr));
  const int need = keff - gt;  // how many keys equal to thr to keep (lowest index first)

  int32_t* dst = idx + grow * topk;
  int out_base = 0, eq_base = 0;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const bool is_eq = key[j] == thr;
    const uint64_t eqm = ballot(is_eq);
    const int eq_rank = eq_base + static_cast<int>(lanes_below(eqm));
    const bool sel = key[j] > thr || (is_eq && eq_rank < need);
    const uint64_t selm = ballot(sel);
    if (sel) dst[out_base + static_cast<int>(lanes_below(selm))] = lane + 64 * j;
    out_base += __popcll(selm);
    eq_base += __popcll(eqm);
  }
  for (int t = keff + lane; t < topk; t += 64) dst[t] = -1;
}

template <int NPER>
hipError_t launch(const float* panel, int32_t* idx, int64_t row0, int64_t rows, int n, int topk,
                  int causal, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  hipLaunchKernelGGL(topk_kernel<NPER>, grid, dim3(256), 0, s, panel, idx, row0, rows, n, topk,
                     causal);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk_select(const float* panel, int32_t* idx, int64_t row0, int64_t rows, int n,
                              int topk, int causal, hipStream_t stream) {
  const int nb = n / kTile;
  if (nb <= 64) return launch<1>(panel, idx, row0, rows, n, topk, causal, stream);
  if (nb <= 128) return launch<2>(panel, idx, row0, rows, n, topk, causal, stream);
  if (nb <= 256) return launch<4>(panel, idx, row0, rows, n, topk, causal, stream);
  if (nb <= 512) return launch<8>(panel, idx, row0, rows, n, topk, causal, stream);
  if (nb <= 1024) return launch<16>(panel, idx, row0, rows, n, topk, causal, stream);
  return launch<32>(panel, idx, row0, rows, n, topk, causal, stream);
}

}  // namespace bsa
