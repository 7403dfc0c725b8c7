// topk_select.hip -- Stage 1 selection from a stored score panel: each query
// keeps its k highest-scoring blocks (nishantmodi.me
// "sparse-attention-triton-bench", section "Stage 2: fine attention": take the
// top-k highest-scoring blocks per query; indices are int32, section "Two
// things I wish I knew").  bsa_forward normally selects inside the coarse
// scoring kernel instead (coarse_score.hip); this kernel serves the
// stage-level entry point and the panel strategy.
//
// Semantics: candidates are all blocks of the query's sequence (all n/64
// blocks of the head unless a block table splits the head into several
// sequences), or in the causal variant those up to the query's own block,
// which is always kept; indices are relative to the sequence's first block.  k_eff =
// min(k, #candidates), where k is the head's budget (one k for all heads
// unless per-head budgets are given; nishantmodi.me
// "sparse-attention-triton-bench", section "What's next": per-head sparsity
// budgets).  Equal scores go to the lower block index and -0 equals
// +0.  Output: the k_eff indices in ascending order, then -1 up to k.
//
// Input: the panel of a chunk of query rows, block-major (panel[beta][row]).
//   k <= 32: one lane per query row (64 rows per wave, 256 contiguous bytes
//     per block across the wave) offers every candidate, in ascending block
//     order, to an exact register top-KL list (topk_list.hpp), KL >= k.
//   k > 32: the whole wave takes one row at a time: lane l holds blocks
//     l + 64 j, a binary radix search over the 32-bit score keys (ballot +
//     popcount per bit, stopping once exactly k_eff keys reach the prefix)
//     finds the k_eff-th largest key T, and ballot / mbcnt prefix counts write
//     the keys above T, then the lowest-index keys equal to T, in ascending
//     block order.
#include "bsa_device.hpp"
#include "bsa_launch.hpp"
#include "topk_list.hpp"

namespace bsa {
namespace {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int KL>
__global__ __launch_bounds__(64) void topk_lane_kernel(const float* __restrict__ panel,
                                                       int32_t* __restrict__ idx, int64_t row0,
                                                       int64_t prows, int n, int topk,
                                                       const HeadBudget budget, int causal,
                                                       const int4* __restrict__ seqtab) {
  const int lane = threadIdx.x;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 64 + lane;  // prows % 64 == 0
  const int64_t grow = row0 + r;
  const RowBlocks rb = row_blocks(seqtab, grow, n, causal);  // the same in all 64 rows
  const int nvalid = rb.hi;
  const int kh = budget.k[(grow / n) % budget.heads];  // the same in all 64 rows
  const int keff = kh < rb.hi - rb.lo ? kh : rb.hi - rb.lo;
  const float* col = panel + r;
  const int forced = causal ? rb.own : -1;

  TopList<KL> l;
  l.init();
  int beta = rb.lo;
  for (; beta + 8 <= nvalid; beta += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = col[static_cast<int64_t>(beta + u) * prows];
#pragma unroll
    for (int u = 0; u < 8; ++u) l.offer(beta + u == forced ? INFINITY : v[u], beta + u);
  }
  for (; beta < nvalid; ++beta) {
    const float v = col[static_cast<int64_t>(beta) * prows];
    l.offer(beta == forced ? INFINITY : v, beta);
  }
  emit_ascending<KL>(l, keff, topk, idx + grow * topk, rb.lo);
}

// Binary radix search for the k-th largest key over NV keys per lane.
// Returns P with #{key >= P} >= k; `early` means exactly k keys are >= P,
// otherwise P is the k-th largest key itself.
template <int NV>
__device__ __forceinline__ uint32_t radix_kth(const uint32_t (&key)[NV], int k, bool& early) {
  uint32_t prefix = 0u;
  early = false;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = prefix | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) cnt += __popcll(ballot(key[j] >= cand));
    if (cnt >= k) {
      prefix = cand;
      if (cnt == k) {
        early = true;
        break;
      }
    }
  }
  return prefix;
}

// One wave per row, rows taken in turn; 4 waves per workgroup of 64 rows.
template <int NPER>
__global__ __launch_bounds__(256) void topk_wave_kernel(const float* __restrict__ panel,
                                                        int32_t* __restrict__ idx, int64_t row0,
                                                        int64_t prows, int n, int topk,
                                                        const HeadBudget budget, int causal,
                                                        const int4* __restrict__ seqtab) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int rr = 0; rr < 16; ++rr) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 64 + wave * 16 + rr;
    const int64_t grow = row0 + r;
    const RowBlocks rb = row_blocks(seqtab, grow, n, causal);
    const int kh = budget.k[(grow / n) % budget.heads];
    const int keff = kh < rb.hi - rb.lo ? kh : rb.hi - rb.lo;
    int32_t* dst = idx + grow * topk;
    uint32_t key[NPER];
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const int e = lane + 64 * j;
      uint32_t kk = 0u;  // not a candidate: below every score
      if (e >= rb.lo && e < rb.hi)
        kk = (causal && e == rb.own) ? 0xffffffffu : order_key(panel[static_cast<int64_t>(e) * prows + r]);
      key[j] = kk;
    }
    bool early;
    const uint32_t P = radix_kth<NPER>(key, keff, early);
    const uint32_t thr = early ? P - 1u : P;  // keys > thr are in; ties at thr fill up
    int gt = 0;
#pragma unroll
    for (int j = 0; j < NPER; ++j) gt += __popcll(ballot(key[j] > thr));
    const int need = keff - gt;
    int out_base = 0, eq_base = 0;
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const bool is_eq = key[j] == thr;
      const uint64_t eqm = ballot(is_eq);
      const int eq_rank = eq_base + static_cast<int>(lanes_below(eqm));
      const bool sel = key[j] > thr || (is_eq && eq_rank < need);
      const uint64_t selm = ballot(sel);
      if (sel) dst[out_base + static_cast<int>(lanes_below(selm))] = lane + 64 * j - rb.lo;
      out_base += __popcll(selm);
      eq_base += __popcll(eqm);
    }
    for (int t = keff + lane; t < topk; t += 64) dst[t] = -1;
  }
}

template <int NPER>
void launch_wave(const float* panel, int32_t* idx, int64_t row0, int64_t rows, int n, int topk,
                 const HeadBudget& hb, int causal, const int4* seqtab, hipStream_t s) {
  hipLaunchKernelGGL((topk_wave_kernel<NPER>), dim3(static_cast<unsigned>(rows / 64)), dim3(256), 0, s,
                     panel, idx, row0, rows, n, topk, hb, causal, seqtab);
}

}  // namespace

hipError_t launch_topk_select(const float* panel, int32_t* idx, int64_t row0, int64_t rows, int n,
                              int topk, const HeadBudget& hb, int causal, hipStream_t s,
                              const int4* seqtab) {
  const dim3 grid(static_cast<unsigned>(rows / 64));
  if (topk <= 8) {
    hipLaunchKernelGGL((topk_lane_kernel<8>), grid, dim3(64), 0, s, panel, idx, row0, rows, n, topk, hb, causal, seqtab);
  } else if (topk <= 16) {
    hipLaunchKernelGGL((topk_lane_kernel<16>), grid, dim3(64), 0, s, panel, idx, row0, rows, n, topk, hb, causal, seqtab);
  } else if (topk <= 32) {
    hipLaunchKernelGGL((topk_lane_kernel<32>), grid, dim3(64), 0, s, panel, idx, row0, rows, n, topk, hb, causal, seqtab);
  } else {
    const int nb = n / kTile;
    if (nb <= 64) launch_wave<1>(panel, idx, row0, rows, n, topk, hb, causal, seqtab, s);
    else if (nb <= 128) launch_wave<2>(panel, idx, row0, rows, n, topk, hb, causal, seqtab, s);
    else if (nb <= 256) launch_wave<4>(panel, idx, row0, rows, n, topk, hb, causal, seqtab, s);
    else if (nb <= 512) launch_wave<8>(panel, idx, row0, rows, n, topk, hb, causal, seqtab, s);
    else if (nb <= 1024) launch_wave<16>(panel, idx, row0, rows, n, topk, hb, causal, seqtab, s);
    else launch_wave<32>(panel, idx, row0, rows, n, topk, hb, causal, seqtab, s);
  }
  return hipGetLastError();
}

}  // namespace bsa
