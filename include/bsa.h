/*
 * bsa.h -- C ABI of libbsa, a two-stage, content-dependent block-sparse
 * attention forward pass for AMD Instinct MI355X (gfx950).
 *
 * The method (nishantmodi.me post "sparse-attention-triton-bench"):
 *   Stage 1 ("Two-stage block indexer", "Stage 1: coarse scoring"): split the
 *     keys into blocks of B, mean-pool each block into a representative, score
 *     every query against every representative, and keep each query's top-k
 *     blocks.  The choice is made at run time, per query and per head.
 *   Stage 2 ("Stage 2: fine attention", "The Triton kernel"): softmax
 *     attention of each query over only the k*B keys of its selected blocks,
 *     with an online softmax (running max m, running sum l, unnormalised
 *     accumulator) so that no score matrix is written to memory.
 * The static mode runs the same fine kernel over a precomputed list of active
 * 64x64 (query tile, key tile) pairs (yayme/CUDA-kernel README: the tile
 * list is built on the CPU and the kernel walks it instead of scanning a
 * mask; masked keys take no part, i.e. score -inf).
 *
 * Conventions shared by every entry point:
 *  - Tensors are row-major [batch][heads][n][d] with d innermost, contiguous,
 *    16-byte aligned, in device memory owned by the caller.  The library never
 *    frees caller memory.
 *  - dtype BSA_BF16: q, k, v hold bfloat16 bit patterns (uint16).  BSA_FP32:
 *    float32.  Outputs are always float32; block indices are always int32.
 *  - "stream" is a hipStream_t (NULL = the null stream).  Work is enqueued on
 *    it and the call returns without waiting: BSA_OK means "validated and
 *    enqueued".  A device fault surfaces at the caller's next synchronisation.
 *  - Validation is synchronous and happens before anything is enqueued; a
 *    failing call enqueues nothing, returns a specific status and leaves a
 *    message readable with bsa_last_error().  Calls never abort or print.
 *  - A handle is not thread-safe: use one handle per host thread / stream.
 *    Two calls on one handle that overlap on different streams race on the
 *    handle's workspace.
 *  - Supported today: block (= tile) 64; d in {64, 128}; ceil(n/64) <= 2048
 *    for the dynamic path.  n need not be a multiple of 64 in bsa_forward,
 *    bsa_forward_budgets, bsa_forward_train, bsa_backward, bsa_fine_forward
 *    and bsa_forward_static: the last block then holds the n mod 64
 *    remaining keys and its representative is their mean (the dynamic calls
 *    run on copies padded to whole blocks, workspace held by the handle,
 *    with the padding keys masked; the static mode reads the sequence in
 *    place).  The stage exports need n a multiple of 64.  Anything else
 *    returns BSA_ERR_UNSUPPORTED.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bsa_handle_s* bsa_handle;

/* A static tile list validated on the host and copied to device memory
 * (bsa_tiles_create).  It belongs to the device of the handle it was made
 * with and stays valid until bsa_tiles_destroy. */
typedef struct bsa_tiles_s* bsa_tiles;

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad scale, misaligned pointer, bad CSR */
  BSA_ERR_UNSUPPORTED = 2,   /* valid request outside what is implemented (d, block, n) */
  BSA_ERR_NO_DEVICE = 3,     /* no HIP device, or the device is not gfx950 */
  BSA_ERR_OUT_OF_MEMORY = 4, /* workspace allocation failed */
  BSA_ERR_LAUNCH = 5         /* the HIP runtime refused a launch or an event/copy call */
} bsa_status;

typedef enum { BSA_FP32 = 0, BSA_BF16 = 1 } bsa_dtype;

/* Stages, for the per-stage timer below. */
typedef enum {
  BSA_STAGE_POOL = 0,    /* block_pool                                         */
  BSA_STAGE_COARSE = 1,  /* coarse_score                                       */
  BSA_STAGE_TOPK = 2,    /* topk_select                                        */
  BSA_STAGE_FINE = 3,    /* sparse_flash_fwd (the MFMA attention kernel)       */
  BSA_STAGE_GATHER_INDEX = 4,   /* block-gather: bucketing of (query, block) pairs */
  BSA_STAGE_GATHER_COMBINE = 5, /* block-gather: merge of per-block partials       */
  BSA_STAGE_COARSE_TOPK = 6,    /* coarse_score and topk_select fused in one kernel  */
  BSA_STAGE_BWD_PREP = 7,       /* backward: per-row lse and delta = dout . out      */
  BSA_STAGE_BWD_INDEX = 8,      /* backward: bucketing of (query, block) pairs       */
  BSA_STAGE_BWD_PAIRS = 9,      /* backward: the MFMA pair kernel (dq, dk, dv parts) */
  BSA_STAGE_BWD_REDUCE = 10,    /* backward: sums of the dq and dk/dv contributions  */
  BSA_STAGE_RAGGED_COPY = 11,   /* n not a multiple of 64: copies to / from padding  */
  BSA_STAGE_STATIC_COMBINE = 12, /* static mode: merge of the items of a cut list     */
  BSA_NUM_STAGES = 13
} bsa_stage;

/* How the dynamic fine stage visits the selected blocks. */
typedef enum {
  /* Group the (query, block) pairs by key block, run 16 pairs per MFMA tile,
   * write split-softmax partials (a normalised output row that also carries
   * the pair's log-sum-exp) and merge them per query.  Every selected pair is
   * computed once.  Default. */
  BSA_FINE_BLOCK_GATHER = 0,
  /* Per query tile (64 rows; 16 or 32 with BSA_OPT_UNION_ROWS), walk the
   * union of the rows' selected blocks with the online softmax in registers,
   * masking each row to its own selection. */
  BSA_FINE_QUERY_TILE = 1,
  /* One wave per query walks the query's own selected blocks with the online
   * softmax on the vector units (nishantmodi.me
   * "sparse-attention-triton-bench", "The Triton kernel": one program per
   * (batch, head, query)); every (query, block) pair reads its block again.
   * For comparison; the slowest of the three on large problems. */
  BSA_FINE_PER_QUERY = 2
} bsa_fine_strategy;

/* How bsa_forward runs stage 1 (the selection is the same either way). */
typedef enum {
  /* For k <= 32: one kernel scores each 64-query tile against every block
   * representative and keeps each query's top k in registers, so the score
   * panel is never stored.  Larger k falls back to BSA_SELECT_PANEL.
   * Default. */
  BSA_SELECT_FUSED = 0,
  /* coarse_score writes the float32 panel (in chunks, see
   * BSA_OPT_PANEL_CHUNK_BYTES), topk_select reads it back. */
  BSA_SELECT_PANEL = 1
} bsa_select_strategy;

/* Tunables for bsa_set_option. */
typedef enum {
  /* Upper bound in bytes of the fp32 coarse-score panel that stage 1 keeps at
   * once; queries are processed in chunks of at most this many bytes of panel.
   * Default 128 MiB.  Minimum one 64-query tile. */
  BSA_OPT_PANEL_CHUNK_BYTES = 0,
  /* bsa_fine_strategy for the dynamic fine stage.  Default BSA_FINE_BLOCK_GATHER. */
  BSA_OPT_FINE_STRATEGY = 1,
  /* Upper bound in bytes of the block-gather partial buffer; query rows are
   * processed in chunks that fit.  Default 1 GiB.  Minimum one 64-query tile. */
  BSA_OPT_FINE_CHUNK_BYTES = 2,
  /* bsa_select_strategy for stage 1 of bsa_forward.  Default BSA_SELECT_FUSED. */
  BSA_OPT_SELECT_STRATEGY = 3,
  /* bsa_forward_static: the most key tiles one work item (one workgroup)
   * takes from a query tile's list; a longer list is cut into several items
   * whose partial results are merged.  0 (default): chosen per call so that
   * there are about two items per compute unit and none is longer than
   * about twice the mean list; a value >= every list length gives one item
   * per query tile. */
  BSA_OPT_STATIC_ITEM_TILES = 4,
  /* Rows per query tile of BSA_FINE_QUERY_TILE: 16, 32 or 64 (default 64). */
  BSA_OPT_UNION_ROWS = 5
} bsa_option;

/* ----------------------------------------------------------- lifetime -- */

/* The lifetime, option, workspace and timing calls are this library's own
 * plumbing: no page defines them.  The pages' interface is the two-stage
 * call with block size B and top-k (nishantmodi.me "sparse-attention-triton-
 * bench", section "Two-stage block indexer") and the README's call on Q, K, V
 * and a mask (yayme/CUDA-kernel README, the usage example); bsa_forward and
 * bsa_forward_static below are those. */

/* Create a handle bound to HIP device `device`.  *out receives the handle.
 * BSA_ERR_NO_DEVICE if there is no HIP device, `device` is out of range, or
 * the device is not gfx950.  The library loads (and this call fails cleanly)
 * on a machine without a GPU. */
bsa_status bsa_create(int device, bsa_handle* out);

/* Free the handle and its workspace.  The caller must make sure no work that
 * uses the handle is still running.  NULL is accepted. */
bsa_status bsa_destroy(bsa_handle h);

/* Static text for a status.  Never NULL. */
const char* bsa_status_string(bsa_status s);

/* Detail of the last failing call on h (or, for h == NULL, of the last
 * failing call on this thread that had no handle).  Never NULL. */
const char* bsa_last_error(bsa_handle h);

/* Set a tunable (see bsa_option).  BSA_ERR_INVALID_ARG for an unknown option
 * or a value out of range. */
bsa_status bsa_set_option(bsa_handle h, int option, int64_t value);

/* Bytes of device workspace the handle holds right now (repr, panel chunk,
 * internal index buffer). */
bsa_status bsa_workspace_bytes(bsa_handle h, size_t* bytes);

/* --------------------------------------------------- dynamic forward -- */

/* Both stages: block_pool -> coarse_score -> topk_select -> sparse_flash_fwd
 * (coarse_score and topk_select fused for k <= 32, see bsa_select_strategy).
 *  q, k, v        device, [batch][heads][n][d], dtype.
 *  out            device, float32 [batch][heads][n][d].
 *  block_idx_out  device, int32 [batch][heads][n][topk] or NULL.  When given,
 *                 it receives each query's selected blocks in ascending order,
 *                 padded with -1 (k_eff = min(topk, #candidate blocks)).  When
 *                 NULL the handle uses an internal buffer.
 *  block          key-block size B; must be 64.
 *  topk           k >= 1; k above the number of candidate blocks keeps them all.
 *  scale          softmax scale (finite, > 0), typically 1/sqrt(d).
 *  causal         0: every block is a candidate.  1: candidates are the blocks
 *                 up to the query's own block, the own block is always kept
 *                 (as one of the k), and inside kept blocks only keys j <= i
 *                 are visible.
 * Coarse scores are q . mean(block keys), unscaled; equal scores go to the
 * lower block index, and -0 equals +0.
 * Range and precision: with bf16 inputs the block-gather fine stage (the
 * default) keeps each (query, block) partial output in fp16, so every |v|
 * must stay below 65504; a larger value makes the affected output rows
 * non-finite (never a finite wrong value).  The fp16 rows (at most 1.5 ulp
 * each, the last mantissa bit of 32 elements carrying the pair's
 * log-sum-exp) and the bf16 probabilities give outputs an absolute error of
 * order 2^-9 * max |v| (about 1e-4 * max |v| measured); for fp32 inputs all
 * of it is fp32.  The same holds for every entry point below that runs the
 * dynamic fine stage on bf16 inputs. */
bsa_status bsa_forward(bsa_handle h, const void* q, const void* k, const void* v,
                       float* out, int32_t* block_idx_out, int batch, int heads,
                       int n, int d, bsa_dtype dtype, int block, int topk,
                       float scale, int causal, void* stream);

/* bsa_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * call makes no hipMalloc, hipFree or other allocation: all its workspace
 * (block representatives, score-panel chunks, the fine stage's bucketing
 * buffers and partial rows) comes from one fixed device array of
 * BSA_NOALLOC_WORKSPACE_BYTES per device, held by the library until the
 * process ends.  The fine stage processes query rows in the largest chunks
 * whose buffers fit.  Results equal bsa_forward's with the same arguments.
 *  block_idx_out  required (the caller provides the index buffer).
 *  n              a multiple of 64 (BSA_ERR_UNSUPPORTED otherwise).
 * A problem whose representatives, or whose smallest fine-stage chunk, do
 * not fit the fixed array returns BSA_ERR_UNSUPPORTED and enqueues nothing.
 * Every call on a device shares that device's array: calls that overlap on
 * one device (different streams, threads or handles) race and give wrong
 * results.  Per-stage timing is not recorded for this call.  Everything else
 * as for bsa_forward. */
#define BSA_NOALLOC_WORKSPACE_BYTES (64u << 20)
bsa_status bsa_forward_noalloc(bsa_handle h, const void* q, const void* k, const void* v,
                               float* out, int32_t* block_idx_out, int batch, int heads,
                               int n, int d, bsa_dtype dtype, int block, int topk,
                               float scale, int causal, void* stream);

/* Like bsa_forward with a top-k budget per head (nishantmodi.me
 * "sparse-attention-triton-bench", section "What's next": each head keeps
 * its own number of blocks, chosen at run time).
 *  head_topk      host, int32 [heads]: head h of every batch keeps
 *                 k_eff = min(head_topk[h], #candidate blocks) blocks;
 *                 1 <= head_topk[h] <= topk_max, else BSA_ERR_INVALID_ARG.
 *                 Read during the call only.
 *  topk_max       row length of block_idx_out: int32
 *                 [batch][heads][n][topk_max], each row's k_eff indices in
 *                 ascending order, then -1.
 *  heads          at most 256 (BSA_ERR_UNSUPPORTED above).
 * Everything else as for bsa_forward; with every head_topk[h] = topk_max
 * the result equals bsa_forward's with topk = topk_max. */
bsa_status bsa_forward_budgets(bsa_handle h, const void* q, const void* k,
                               const void* v, float* out, int32_t* block_idx_out,
                               int batch, int heads, int n, int d,
                               bsa_dtype dtype, int block,
                               const int32_t* head_topk, int topk_max,
                               float scale, int causal, void* stream);

/* ------------------------------------------------------------ training -- */

/* The forward for training: bsa_forward (or bsa_forward_budgets) that also
 * stores what bsa_backward needs.
 *  block_idx_out  device, int32 [batch][heads][n][topk], required.
 *  lse_out        device, float32 [batch][heads][n], required, 4-byte aligned:
 *                 per query row log(sum_j exp(scale * q.k_j)) over its visible
 *                 keys (natural log).
 *  head_topk      host, int32 [heads], or NULL for topk on every head; as in
 *                 bsa_forward_budgets with topk_max = topk.
 * Everything else as for bsa_forward. */
bsa_status bsa_forward_train(bsa_handle h, const void* q, const void* k,
                             const void* v, float* out, int32_t* block_idx_out,
                             float* lse_out, int batch, int heads, int n, int d,
                             bsa_dtype dtype, int block, const int32_t* head_topk,
                             int topk, float scale, int causal, void* stream);

/* Backward of the fine stage (nishantmodi.me "sparse-attention-triton-bench",
 * section "What's next": a backward pass through the softmax-weighted sum over
 * the selected blocks, FlashAttention-2's backward as the dense model).  The
 * selection is a discrete choice and gets no gradient: block_idx is held
 * fixed, and q, k, v get the gradients of softmax attention over each row's
 * visible keys (its selected blocks; j <= i when causal):
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
 *   dv_j = sum_i p_ij dout_i,  ds_ij = p_ij (dout_i . v_j - dout_i . out_i),
 * with p_ij = exp(scale q_i.k_j - lse_i) recomputed from lse.
 *  q, k, v        device, as passed to bsa_forward_train.
 *  out, lse, block_idx  device, as written by bsa_forward_train for the same
 *                 q, k, v, topk, scale and causal (row length topk).
 *  dout           device, float32 [batch][heads][n][d]: gradient of out.
 *  dq, dk, dv     device, float32 [batch][heads][n][d], written (every
 *                 element; keys no row sees get 0).
 * Pointers 16-byte aligned except block_idx and lse (4).  No floating-point
 * atomics: dq is the same bit for bit on every call (each (query, block)
 * contribution is computed alone and they are summed in slot order); dk and
 * dv sum the pairs of a key block in the order the bucketing lists them,
 * which its integer atomics set, so two calls can differ in the last bits.
 * Workspace grows with topk * n (bounded by BSA_OPT_FINE_CHUNK_BYTES, the
 * rows being processed in chunks). */
bsa_status bsa_backward(bsa_handle h, const void* q, const void* k, const void* v,
                        const float* out, const float* dout,
                        const int32_t* block_idx, const float* lse, float* dq,
                        float* dk, float* dv, int batch, int heads, int n, int d,
                        bsa_dtype dtype, int block, int topk, float scale,
                        int causal, void* stream);

/* --------------------------------------------------- variable lengths -- */

/* A batch of sequences of different lengths (yayme/CUDA-kernel README, file
 * table: the correctness tests include lengths that are not a multiple of
 * the tile; nishantmodi.me "sparse-attention-triton-bench", section "Stage 1:
 * coarse scoring": the blocks are those of each sequence's own keys).
 * Sequence i is rows cu_seqlens[i] .. cu_seqlens[i + 1] - 1 of every head,
 * and it is attended to on its own: its key blocks start at its first row
 * (the last one may be partial and is then pooled over the keys it has), a
 * query's candidates are the blocks of its sequence only, and in the causal
 * variant position j <= i counts within the sequence.
 *  q, k, v        device, [heads][total][d], dtype, total = cu_seqlens[nseq]
 *                 (each head's rows of all sequences, one after the other).
 *  out            device, float32 [heads][total][d].
 *  block_idx_out  device, int32 [heads][total][topk] or NULL: each query's
 *                 selected blocks numbered from its sequence's first block
 *                 (0 = rows cu_seqlens[i] .. cu_seqlens[i] + 63), ascending,
 *                 -1 padded; k_eff = min(budget, blocks of the sequence up to
 *                 the query's own block when causal).
 *  lse_out        device, float32 [heads][total] or NULL: as for
 *                 bsa_forward_train (what bsa_backward_varlen needs).
 *  cu_seqlens     host, int32 [nseq + 1]: cu_seqlens[0] = 0, non-decreasing
 *                 (empty sequences allowed), total >= 1; read during the call
 *                 only.  Else BSA_ERR_INVALID_ARG.
 *  head_topk      host, int32 [heads] or NULL: per-head budgets as for
 *                 bsa_forward_budgets, with topk the index row length.
 * The sequences padded to whole 64-row blocks may take at most 2048 blocks
 * per head (BSA_ERR_UNSUPPORTED).  Everything else as for bsa_forward; each
 * sequence's result equals bsa_forward's on that sequence alone. */
bsa_status bsa_forward_varlen(bsa_handle h, const void* q, const void* k,
                              const void* v, float* out, int32_t* block_idx_out,
                              float* lse_out, const int32_t* cu_seqlens, int nseq,
                              int heads, int d, bsa_dtype dtype, int block,
                              const int32_t* head_topk, int topk, float scale,
                              int causal, void* stream);

/* bsa_backward for a batch laid out as for bsa_forward_varlen: out, lse and
 * block_idx as that call wrote them (lse_out and block_idx_out given), dout,
 * dq, dk, dv float32 [heads][total][d].  Everything else as for
 * bsa_backward. */
bsa_status bsa_backward_varlen(bsa_handle h, const void* q, const void* k,
                               const void* v, const float* out, const float* dout,
                               const int32_t* block_idx, const float* lse, float* dq,
                               float* dk, float* dv, const int32_t* cu_seqlens,
                               int nseq, int heads, int d, bsa_dtype dtype, int block,
                               int topk, float scale, int causal, void* stream);

/* Stage 2 alone on caller-supplied selections (nishantmodi.me
 * "sparse-attention-triton-bench", sections "Stage 2: fine attention" and "The
 * Triton kernel": each query attends only to the keys of the blocks it
 * selected, with an online softmax; the block ids are int32, section "Two
 * things I wish I knew").
 *  block_idx      device, int32 [batch][heads][n][topk] (the layout of
 *                 block_idx_out above); each row must hold distinct indices;
 *                 entries outside [0, ceil(n/block)), and in causal mode
 *                 blocks after the query's own block, count as padding.
 * Everything else as for bsa_forward; the output is the same as
 * bsa_forward's for that selection.  Useful to test or reuse a selection. */
bsa_status bsa_fine_forward(bsa_handle h, const void* q, const void* k,
                            const void* v, float* out, const int32_t* block_idx,
                            int batch, int heads, int n, int d, bsa_dtype dtype,
                            int block, int topk, float scale, int causal,
                            void* stream);

/* ---------------------------------------------------- stage 1 pieces -- */

/* block_pool alone (nishantmodi.me "sparse-attention-triton-bench", section
 * "Stage 1: coarse scoring": the keys are split into blocks of B and each
 * block is mean-pooled into one representative vector).
 *  k              device, [batch][heads][n][d], dtype.
 *  repr_out       device, float32 [batch][heads][n/B][d], 16-byte aligned:
 *                 repr_out[b][h][beta][:] = mean of keys beta*B .. beta*B+B-1,
 *                 summed in float32.
 *  n              a multiple of 64 (BSA_ERR_UNSUPPORTED otherwise); other
 *                 arguments as for bsa_forward. */
bsa_status bsa_block_pool(bsa_handle h, const void* k, float* repr_out,
                          int batch, int heads, int n, int d, bsa_dtype dtype,
                          int block, void* stream);

/* coarse_score alone (nishantmodi.me "sparse-attention-triton-bench", section
 * "Stage 1: coarse scoring": every query is scored against every block
 * representative, Q times the transposed representatives, O(N * N/B)).
 *  q              device, [batch][heads][n][d], dtype.
 *  repr           device, float32 [batch][heads][n/B][d] as bsa_block_pool
 *                 writes it.
 *  panel_out      device, float32, block-major: with rows = batch*heads*n and
 *                 row = (b*heads + h)*n + i,
 *                 panel_out[beta * rows + row] = q_i . repr[b][h][beta]
 *                 (beta < n/B), unscaled.  In causal mode entries with
 *                 beta > i/B are unspecified.
 * n a multiple of 64; errors as for bsa_forward.  The caller owns the panel
 * (batch*heads*n*(n/64)*4 bytes). */
bsa_status bsa_coarse_score(bsa_handle h, const void* q, const float* repr,
                            float* panel_out, int batch, int heads, int n, int d,
                            bsa_dtype dtype, int block, int causal, void* stream);

/* topk_select alone (nishantmodi.me "sparse-attention-triton-bench", section
 * "Stage 2: fine attention": each query keeps its top-k highest-scoring
 * blocks; the ids are int32, section "Two things I wish I knew").
 *  panel          device, float32, block-major as bsa_coarse_score writes it.
 *  block_idx_out  device, int32 [batch][heads][n][topk]: per row the selection
 *                 exactly as described for bsa_forward (ties to the lower
 *                 block, -0 equal to +0, ascending, -1 padded; causal: the own
 *                 block kept, later blocks not candidates).
 * n a multiple of 64; errors as for bsa_forward. */
bsa_status bsa_topk_select(bsa_handle h, const float* panel,
                           int32_t* block_idx_out, int batch, int heads, int n,
                           int block, int topk, int causal, void* stream);

/* ------------------------------------------------------ static forward -- */

/* The static mode runs the fine attention of bsa_fine_forward over a fixed
 * list of active (64-query tile, 64-key tile) pairs instead of a selection
 * (yayme/CUDA-kernel README: precompute the active tile list on the CPU and
 * skip inactive tiles instead of scanning the mask in the kernel; infra.bea.ai
 * "Block-Sparse & Linear Attention Kernels", section 4: a compressed list of
 * active blocks per row as the mask representation).  Format: CSR over query
 * tiles.  With nt = ceil(n/64):
 *  row_ptr   int32 [nt + 1]: row_ptr[0] = 0, non-decreasing, row_ptr[nt] = nnz;
 *            query tile t (rows 64t .. min(64t+63, n-1)) visits key tiles
 *            col[row_ptr[t] .. row_ptr[t+1]).
 *  col       int32 [nnz]: key-tile ids in [0, nt), strictly increasing inside
 *            each query tile's range.
 *  rowmask   uint64 [nnz][64] or NULL: bit c of entry (p, r) says whether
 *            query row r of the tile sees key c of tile col[p]; bits of keys
 *            at or past n must be clear.  NULL means every listed tile is
 *            fully visible (keys past n excepted).
 * A key that is not visible takes no part in the softmax (score -inf, the
 * README's note on its v1 bug); a row that sees no key gets zeros. */

/* Validate a tile list held in HOST memory and copy it to the device of h.
 *  n, tile   sequence length (>= 1, need not be a multiple of 64) and tile
 *            size (must be 64: BSA_ERR_UNSUPPORTED otherwise).
 *  row_ptr, col, rowmask, nnz   as above, host memory, read during the call
 *            only.
 *  out       receives the list; free it with bsa_tiles_destroy.
 * Every rule above is checked: a malformed list returns BSA_ERR_INVALID_ARG
 * (bsa_last_error(h) names the first broken rule) and creates nothing.
 * BSA_ERR_OUT_OF_MEMORY if the device copy cannot be allocated.  Blocks
 * until the copy is done. */
bsa_status bsa_tiles_create(bsa_handle h, int n, int tile, const int32_t* row_ptr,
                            const int32_t* col, const uint64_t* rowmask, int64_t nnz,
                            bsa_tiles* out);

/* Free a tile list.  No work that uses it may still be running.  NULL is
 * accepted. */
bsa_status bsa_tiles_destroy(bsa_tiles t);

/* Fine attention over a tile list, the same list for every batch and head.
 *  q, k, v, out, batch, heads, n, d, dtype, scale   as for bsa_forward; n
 *            must equal the n the list was made for (BSA_ERR_INVALID_ARG).
 *  tile      must be 64 (BSA_ERR_UNSUPPORTED otherwise).
 *  tiles     from bsa_tiles_create with the same handle's device.
 * Work: query tiles whose list is longer than the item size (see
 * BSA_OPT_STATIC_ITEM_TILES) are cut into several work items, heaviest first
 * (infra.bea.ai, section 4, the challenges table: load imbalance answered by
 * dynamic block scheduling); their partials go to handle workspace and are
 * merged.  The first call with a new item size builds that schedule on the
 * host and copies it to the device (synchronously, once). */
bsa_status bsa_forward_static(bsa_handle h, const void* q, const void* k,
                              const void* v, float* out, int batch, int heads,
                              int n, int d, bsa_dtype dtype, int tile,
                              bsa_tiles tiles, float scale, void* stream);

/* Host helper: tile list of a dense element mask (same source as above).
 * mask is host uint8 [n][n] (nonzero = visible).  row_ptr: host int32
 * [ceil(n/64) + 1].  col: host int32 [*nnz_inout] or NULL; rowmask: host
 * uint64 [*nnz_inout][64] or NULL.  With col == NULL only counts: *nnz_inout
 * receives the number of active tiles.  Otherwise *nnz_inout must be >= that
 * number on entry (BSA_ERR_INVALID_ARG) and receives it on return.  tile must
 * be 64; any n >= 1. */
bsa_status bsa_tiles_from_mask(const uint8_t* mask, int n, int tile,
                               int32_t* row_ptr, int32_t* col,
                               uint64_t* rowmask, int64_t* nnz_inout);

/* Host helper: the same for the window+stride pattern (yayme/CUDA-kernel
 * README, the sparsity pattern: query i sees key j iff |i-j| <= window or
 * j mod stride == 0) without materialising the mask. */
bsa_status bsa_tiles_window_stride(int n, int window, int stride, int tile,
                                   int32_t* row_ptr, int32_t* col,
                                   uint64_t* rowmask, int64_t* nnz_inout);

/* Host helper: BSA_OK iff (row_ptr, col) satisfies the rules above for n and
 * tile (the row masks are not looked at); else the status bsa_tiles_create
 * would return. */
bsa_status bsa_tiles_validate(const int32_t* row_ptr, const int32_t* col,
                              int64_t nnz, int n, int tile);

/* ------------------------------------------------------------ timing -- */

/* Enable (1) or disable (0) per-stage timing.  While enabled every kernel
 * launch is bracketed by two HIP events on the launch stream. */
bsa_status bsa_profile_enable(bsa_handle h, int on);

/* Wait for the recorded events and return, per bsa_stage, the summed kernel
 * time in milliseconds (ms[BSA_NUM_STAGES]) and the number of launches
 * (launches[BSA_NUM_STAGES], may be NULL).  reset != 0 clears the record. */
bsa_status bsa_profile_read(bsa_handle h, double* ms, int64_t* launches,
                            int reset);

/* The fused selection (bsa_forward and the entry points built on it, with
 * BSA_SELECT_FUSED and k <= 32) keeps each query's candidates in a fixed
 * number of slots per lane (8 for k <= 8, 16 for k <= 16, 32 for k <= 32,
 * except 24 for bf16 inputs at d = 128).
 * A 64-query workgroup in which some lane has more candidates walks the
 * scores a second time with a higher bound; if a lane overflows again, it
 * redoes the walk with exact per-lane top-k lists.  Every path gives the same
 * answer; the later ones are slower.  This writes, for this handle since it
 * was created or last reset, counts[0] = workgroups that walked a second
 * time and counts[1] = workgroups that took the exact redo (reset != 0
 * clears both after reading).  It waits for all work on the handle's device.
 * Errors: INVALID_ARG for a NULL argument, LAUNCH if the device reports an
 * error. */
bsa_status bsa_select_fallbacks(bsa_handle h, int64_t* counts, int reset);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
