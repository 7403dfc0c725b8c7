// topk_list.hpp -- exact running top-k of (score, block) pairs kept in
// registers, shared by the selection kernels.
//
// Ranking (nishantmodi.me "sparse-attention-triton-bench", section "Stage 2:
// fine attention": each query keeps its k highest-scoring blocks): higher
// score first; equal scores (with -0 equal to +0) to the lower block index.
// The causal own block, which is always kept, enters with score +inf.
//
// TopList keeps the KL best entries offered so far, sorted: v[0] >= v[1] >=
// ..., equal values in ascending block order; empty slots hold -inf with
// block -1.  Entries must be offered in ascending block order: then a new
// entry belongs right after the last slot whose value is >= its own, so its
// place is p = the first j with x > v[j] (strict), slots p.. shift down by one
// and the last falls off.  The masks x > v[j] are monotone in j, and each
// slot takes its new value from itself, the new entry or its upper neighbour:
// one compare and four selects per slot, with no carried chain.
#pragma once

#include "bsa_device.hpp"

namespace bsa {

template <int KL>
struct TopList {
  float v[KL];
  int b[KL];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int j = 0; j < KL; ++j) {
      v[j] = -INFINITY;
      b[j] = -1;
    }
  }
  // A score of -inf or NaN is never kept.  Slots are updated from the bottom
  // up, so only two compare masks are live at a time.
  __device__ __forceinline__ void offer(float x, int beta) {
    bool below = x > v[KL - 1];
#pragma unroll
    for (int j = KL - 1; j >= 1; --j) {
      const bool above = x > v[j - 1];
      v[j] = above ? v[j - 1] : (below ? x : v[j]);
      b[j] = above ? b[j - 1] : (below ? beta : b[j]);
      below = above;
    }
    v[0] = below ? x : v[0];
    b[0] = below ? beta : b[0];
  }
};

// Write the first `keff` blocks of a sorted list, less `base` (the first
// block of the query's sequence), in ascending order to dst[0 .. keff), then
// -1 up to dst[topk - 1].  Position of an entry = number of selected entries
// with a smaller block index.
template <int KL>
__device__ __forceinline__ void emit_ascending(const TopList<KL>& l, int keff, int topk,
                                               int32_t* __restrict__ dst, int base = 0) {
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    if (j < keff) {
      int pos = 0;
#pragma unroll
      for (int t = 0; t < KL; ++t) pos += (t < keff && l.b[t] < l.b[j]) ? 1 : 0;
      dst[pos] = l.b[j] - base;
    }
  }
  for (int t = keff; t < topk; ++t) dst[t] = -1;
}

}  // namespace bsa
