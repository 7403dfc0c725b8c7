// bsa_launch.hpp -- host-side launchers of the gfx950 kernels.  Each kernel
// file defines its launcher; the C ABI (bsa_api.cpp) validates arguments and
// calls these.  Launchers assume validated arguments: n % 64 == 0, d in
// {64, 128}, n / 64 <= 2048 where stated, 16-byte aligned pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa.h"

namespace bsa {

// block_pool: k [bh][n][d] -> repr float [bh][n/64][d] (if repr != NULL) and
// the three-term bf16 split of each representative, split [bh][3][n/64][d]
// (if split != NULL).  seqtab (nullable): the block table of sequences
// padded to whole blocks (bsa_device.hpp); a block with fewer than 64 keys
// is the mean of those.
//
// Every `seqtab` below is that table: n / 64 entries in device memory, or
// NULL for one sequence of n whole-block rows per head.
hipError_t launch_block_pool(const void* k, float* repr, uint16_t* split, int64_t bh, int n, int d,
                             bsa_dtype dtype, hipStream_t stream, const int4* seqtab = nullptr);

// The split buffer: the three bf16 planes [bh][3][n/64][d], then per block
// the 2-norm of its hi term [bh][n/64] (fp32, rounded up), whose largest
// value over a head the fused selection's first pass uses to bound its error.
inline size_t split_buffer_bytes(int64_t bh, int nb, int d) {
  return static_cast<size_t>(bh) * nb * d * 3 * 2 + static_cast<size_t>(bh) * nb * 4;
}
inline float* split_norms(uint16_t* split, int64_t bh, int nb, int d) {
  return reinterpret_cast<float*>(split + static_cast<size_t>(bh) * nb * d * 3);
}

// Sequences whose lengths are not multiples of 64 run on copies padded to
// whole blocks.  pad: dst [slices][n_pad] rows from src [slices][src_rows]
// rows, row r of a slice taking caller row seqtab[r / 64].w + r % 64 when
// r % 64 < seqtab[r / 64].z, else `fill` in every 32-bit word.  unpad: the
// inverse, for the rows that exist.  Rows are `words` 32-bit words.
hipError_t launch_pad_rows(const void* src, void* dst, int64_t slices, int src_rows, int n_pad, int words,
                           uint32_t fill, const int4* seqtab, hipStream_t stream);
hipError_t launch_unpad_rows(const void* src, void* dst, int64_t slices, int src_rows, int n_pad, int words,
                             const int4* seqtab, hipStream_t stream);

// coarse_score over panel rows [row0, row0 + rows) of the flattened
// [bh * n] query rows; row0 and rows multiples of 64.  panel row r holds
// query row0 + r, nb = n / 64 columns, block-major: panel[beta * rows + r].
hipError_t launch_coarse_score(const void* q, const float* repr, float* panel, int64_t row0,
                               int64_t rows, int n, int d, bsa_dtype dtype, int causal,
                               hipStream_t stream);

// Selection budgets: the query rows of (batch, head) bh keep
// k[bh % heads] blocks; a uniform budget is heads = 1.  Passed by value as a
// kernel argument.  Index rows have `topk` (>= every k) entries, -1 padded.
constexpr int kMaxBudgetHeads = 256;
struct HeadBudget {
  int heads;
  int32_t k[kMaxBudgetHeads];
};

// coarse_score and topk_select in one kernel (topk <= 32) over all `rows`
// query rows: idx[row * topk + t], no panel.  Representatives: for bf16
// inputs the split form from block_pool (repr_split), for fp32 inputs the
// float32 repr.  Candidates: the blocks of the query's sequence; indices
// relative to its first block.  fallbacks (may be null): two device counters;
// a workgroup adds 1 to [0] when it walks the candidates a second time and to
// [1] when it takes the exact fallback.  When select_uses_repair(d, dtype,
// topk), the exact fallback runs in a second kernel launched after the first
// and needs repair_counters (two device ints, zero when the handle was made,
// owned by the caller, the same for every call of a handle), repair_list
// (rows / 64 ints of workspace) and the call's parity (0/1, flipped by the
// caller for every such call; calls must not overlap).  warm (nullable): the
// V the fine stage will read, laid out like q.  When it fits the Infinity
// Cache with room to spare (kWarmMaxBytes) each workgroup also reads its own
// rows of it, so V arrives while this kernel leaves HBM nearly idle instead
// of on the attention kernel's first touch.
inline bool select_uses_repair(int d, bsa_dtype dtype, int topk) {
  return d == 128 && dtype == BSA_BF16 && topk > 16;
}
hipError_t launch_coarse_select(const void* q, const float* repr, const uint16_t* repr_split,
                                int32_t* idx, int64_t rows, int n, int d, bsa_dtype dtype,
                                int topk, const HeadBudget& budget, int causal, hipStream_t stream,
                                const int4* seqtab = nullptr, int32_t* fallbacks = nullptr,
                                int32_t* repair_counters = nullptr, int32_t* repair_list = nullptr,
                                int repair_parity = 0, const void* warm = nullptr);
// V is read ahead only up to this size: Q and K (as large) and the
// bucketing's pair lists also pass through the 256 MB cache before the
// attention kernel runs, and would evict a larger V again first.
constexpr int64_t kWarmMaxBytes = int64_t(64) << 20;
constexpr int kFusedSelectMaxK = 32;

// topk_select over panel rows [row0, row0 + rows): idx[(row0 + r) * topk + t].
hipError_t launch_topk_select(const float* panel, int32_t* idx, int64_t row0, int64_t rows, int n,
                              int topk, const HeadBudget& budget, int causal, hipStream_t stream,
                              const int4* seqtab = nullptr);

// sparse_flash_fwd, dynamic: per query tile of `rows` rows (16, 32 or 64)
// the union of its rows' selected blocks, each row masked to its own
// selection.  lse (nullable): per row log-sum-exp of the scaled scores,
// natural log.
hipError_t launch_sparse_flash_dynamic(const void* q, const void* k, const void* v, float* out,
                                       float* lse, const int32_t* idx, int64_t bh, int n, int d,
                                       int topk, float scale, int causal, bsa_dtype dtype,
                                       hipStream_t stream, const int4* seqtab = nullptr, int rows = 64);

// sparse_flash_fwd, per query: one wave per query row walks the row's
// selected blocks in slot order with an online softmax on the vector units
// (no tile sharing between queries).  lse as above.
hipError_t launch_sparse_flash_per_query(const void* q, const void* k, const void* v, float* out,
                                         float* lse, const int32_t* idx, int64_t rows, int n, int d,
                                         int topk, float scale, int causal, bsa_dtype dtype,
                                         hipStream_t stream, const int4* seqtab = nullptr);

// sparse_flash_fwd, static tile list, run as host-scheduled work items (each
// at most S key tiles of one query tile, heaviest first), then a merge of the
// query tiles whose list was cut into several items.
struct StaticLaunch {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  float* out = nullptr;
  int64_t bh = 0;               // batch * heads (the list is the same for each)
  int n = 0, d = 0;             // n: rows per head (need not be a multiple of 64)
  bsa_dtype dtype = BSA_FP32;
  float scale = 0.f;
  const int32_t* col = nullptr;       // [nnz] key tile of each list entry
  const uint64_t* rowmask = nullptr;  // [nnz][64] or NULL (every listed tile fully visible)
  const int4* items = nullptr;  // [nitems] {query tile, first entry, entries, slot or -1}
  int64_t nitems = 0;
  const int4* split = nullptr;  // [nsplit] {query tile, first slot, slots}
  int64_t nsplit = 0;
  int nslots = 0;               // partial slots per (batch, head)
  float* part = nullptr;        // [bh][nslots][64][d]  normalised partial rows
  float* part_lse = nullptr;    // [bh][nslots][64]     their log2-domain log-sum-exp
};
hipError_t launch_sparse_flash_static(const StaticLaunch& a, hipStream_t stream);
hipError_t launch_static_combine(const StaticLaunch& a, hipStream_t stream);  // no-op when nothing is split

// sparse_flash_fwd, block-gather strategy: pairs grouped by key block,
// split-softmax partials, merged per query.  Three launch groups per chunk of
// query rows [row0, row0 + rows) (row0, rows multiples of 64).
struct GatherWorkspace {
  int32_t* count = nullptr;    // [buckets]      buckets = heads spanned by a chunk * n/64; zero
                               // between bucketings (the scan kernel clears what it read)
  int64_t count_words = 0;     // > 0: clear count[0 .. count_words) first (its contents unknown)
  int32_t* offsets = nullptr;  // [buckets + 1]
  int32_t* items = nullptr;    // [buckets + 1]
  int4* item_rec = nullptr;    // [gather_grid(...)]  per-workgroup work-item records
  int32_t* rank = nullptr;     // [chunk pairs]  pairs = rows * topk
  int2* rec = nullptr;         // [chunk pairs]  block-ordered {pair, block << 21 | rank} records
  int32_t* wg_valid = nullptr; // [chunk rows / 64]  valid pairs per bucketing workgroup
  int32_t* list = nullptr;     // [chunk pairs]
  // [chunk pairs][d]  fp16 for bf16 inputs, fp32 for fp32 inputs; the low bits of
  // elements 0 .. 31 of a row hold the pair's log2-domain log-sum-exp (fp32 bits)
  void* partial_o = nullptr;
};

// Pairs per work item of the forward attention kernel: 512 for bf16 inputs
// at d = 64 (measured at N = 32k: attention 0.189 ms against 0.201 at 256;
// fewer key-block stagings per pair), else 256 (at d = 128, 512 pairs take
// the kernel to fewer waves per SIMD: 4.07 against 3.26 ms on the long
// causal workload; fp32 operands are twice the registers).
constexpr int gather_item_pairs(int d, bsa_dtype dtype) { return d == 64 && dtype == BSA_BF16 ? 512 : 256; }

struct GatherArgs {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  float* out = nullptr;
  float* lse = nullptr;  // nullable: per row log-sum-exp (natural log), from the combine
  const int32_t* idx = nullptr;
  int n = 0, d = 0, topk = 0, causal = 0;
  const int4* seqtab = nullptr;  // block table (sequences padded to whole blocks) or NULL
  float scale = 0.f;
  bsa_dtype dtype = BSA_FP32;
  int qsegs = 1;  // query segments per head (gather_segments); buckets = heads x qsegs x n/64
  int item_pairs = 256;  // pairs per work item made by the bucketing (gather_item_pairs for the forward)
  GatherWorkspace ws;
};

// Query segments per head for the bucketing: the pairs of one (head, key
// block) are split by query range so that the work items of one segment,
// which run together, gather query rows from at most 2 MB of Q.  Forward
// only: the backward buckets by (head, block) (measured at N = 32k: 0.69 ms
// with one segment per head, 0.73 with the forward's two, 0.93 with four;
// its per-item dk, dv partials grow with the segments while its gathered Q
// and dO rows hit little in L2 at any of these sizes).
int gather_segments(int n, int d, int topk, bsa_dtype dtype);

size_t gather_pair_bytes(int d, bsa_dtype dtype);  // partial bytes per (query, block) pair
// Work-item slots (workgroups of the kernels that run the items).
int64_t gather_grid(int64_t rows, int topk, int64_t nbuckets, int item_pairs);
hipError_t launch_gather_index(const GatherArgs& a, int64_t row0, int64_t rows, hipStream_t s);
hipError_t launch_gather_partial(const GatherArgs& a, int64_t row0, int64_t rows, hipStream_t s);
hipError_t launch_gather_combine(const GatherArgs& a, int64_t row0, int64_t rows, hipStream_t s);

// Backward of the fine stage with the selection held fixed, on the
// bucketing of the block-gather forward with one query segment per head (one
// work item = up to bwd_item_pairs(d) pairs of one (head, key block) bucket).
// d = 64: 2048 pairs, so a bucket at N = 32k is one item (fewest per-item
// dk, dv partials); d = 128: 1024 (measured on the long causal workload:
// 11.8 ms at 512, 11.2 at 1024, 12.3 at 2048, where long items leave tails).
constexpr int bwd_item_pairs(int d) { return d == 64 ? 2048 : 1024; }

struct BackwardArgs {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const float* out = nullptr;   // forward output [bh][n][d]
  const float* dout = nullptr;  // incoming gradient [bh][n][d]
  const float* lse = nullptr;   // forward log-sum-exp [bh][n]
  const int32_t* idx = nullptr;
  float* dq = nullptr;
  float* dk = nullptr;
  float* dv = nullptr;
  int n = 0, d = 0, topk = 0, causal = 0;
  const int4* seqtab = nullptr;  // block table (sequences padded to whole blocks) or NULL
  float scale = 0.f;
  bsa_dtype dtype = BSA_FP32;
  int qsegs = 1;
  float2* ld = nullptr;      // [bh * n] (lse * log2(e), sum_d dout * out)
  uint16_t* dout_b = nullptr; // [bh * n][d] dout rounded to bf16 (bf16 inputs only)
  float* dq_part = nullptr;  // [chunk pairs][d]  per-pair dq contributions (bf16 for bf16 inputs)
  float* dkv_part = nullptr; // [work items][2][64][d]  per-item dk, dv contributions
  GatherWorkspace ws;        // bucketing (count .. list); partial_o unused
};

// ld for all `rows` query rows.
hipError_t launch_bwd_prep(const BackwardArgs& a, int64_t rows, hipStream_t s);
// Per chunk of query rows [row0, row0 + rows), after launch_gather_index on
// the chunk: the pair kernel, then dq of the chunk's rows and dk, dv of the
// key blocks of the heads the chunk spans (added to what an earlier chunk
// wrote for the head when the head began before row0).
hipError_t launch_bwd_pairs(const BackwardArgs& a, int64_t row0, int64_t rows, hipStream_t s);
hipError_t launch_bwd_dq(const BackwardArgs& a, int64_t row0, int64_t rows, hipStream_t s);
hipError_t launch_bwd_dkv(const BackwardArgs& a, int64_t row0, int64_t rows, hipStream_t s);

// The fixed workspace of bsa_forward_noalloc: a device array of
// kNoAllocScratchBytes per device (noalloc.hip).  noalloc_scratch returns its
// device address on `device`, which must be the current device on the first
// call for that device (the address is looked up once and kept).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(int device, void** out);

}  // namespace bsa
