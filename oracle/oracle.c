/*
 * oracle.c -- plain, slow, fp64 CPU reference for the two-stage,
 * content-dependent block-sparse attention forward pass and for the static
 * window+stride pattern run through the same fine attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code.  It shares no
 * code, header, table or helper with the HIP library, and the HIP library
 * never calls it.
 *
 * What it follows (pages as published; section names in quotes):
 *
 *  [P1] the nishantmodi.me post "sparse-attention-triton-bench", section
 *       "Two-stage block indexer":
 *       Stage 1 splits the keys into blocks of B, mean-pools each block into a
 *       representative vector, and scores every query against every
 *       representative (Q times the transposed representatives), which costs
 *       O(N * N/B).  Stage 2 takes each query's top-k highest-scoring blocks
 *       and runs dense attention over only those k*B keys.  The selection is
 *       per query (and per head, section "What's next").
 *  [P1] same page, section "The Triton kernel": the fine stage is ordinary
 *       softmax attention over the selected keys.  Here it is computed with a
 *       plain two-pass softmax (max, then exp/sum), deliberately NOT the online
 *       update the GPU kernel uses, so the two are algorithmically independent.
 *  [P2] "yayme/CUDA-kernel" README, section on the sparsity pattern: query i
 *       attends key j iff |i - j| <= w or j mod s == 0; masked keys must score
 *       -inf (the README's note on its v1 bug, where they scored 0).
 *
 * Readings taken where the pages are silent (each is repeated at its use):
 *  R1  mean, not sum, and no softmax scale in the coarse score: ranking is
 *      unaffected by a positive factor, so the plainest reading is used.
 *  R2  ties in the coarse score go to the lower block index; -0 equals +0.
 *  R3  k_eff = min(k, number of candidate blocks); indices are emitted in
 *      ascending block order and padded with -1 up to k.
 *  R4  causal variant: candidates are blocks <= the query's own block, the own
 *      block is always kept (it is one of the k: its score is taken as +inf),
 *      and inside the kept blocks only keys j <= i are visible.
 *  R5  a trailing partial block (n not a multiple of B) is pooled as the mean
 *      of its valid keys.
 *  R6  a row with no visible key gets an all-zero output.
 *
 * Layout: every tensor is [bh][n][d] row-major, bh = batch*heads flattened,
 * inputs are the exact float32 values the GPU sees (bf16 inputs are passed as
 * their float32 widening, which is exact); all arithmetic is fp64.
 * "rows" are flattened query rows r = bh_index*n + i.
 *
 * Every function returns 0 on success, a negative value on bad arguments.
 *
 * Pins (tests/test_oracle_pins.py): pooling by column sums and a hand example;
 * scores by numpy's matrix product; selection by pairwise rank with exact
 * ties, by max-sum subset enumeration, by a signed-zero case and a causal
 * brute force; fine attention by textbook dense (and dense causal) attention,
 * single-block attention, constant-V / zero-scale / block-order invariants and
 * two hand-worked examples; the static mask by a hand-written 8x8 case and
 * closed-form pair and tile counts; masked attention by textbook masked
 * softmax; visible pairs by the page's printed FLOP and token counts.  No
 * function here is left parity-unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_EXPORT __attribute__((visibility("default")))

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Stage 1, pooling [P1 "Two-stage block indexer"]: repr[bh][beta][:] is the
 * mean of the keys of block beta (reading R5 for a partial last block). */
ORACLE_EXPORT int oracle_pool(const float* k, int64_t bh, int64_t n, int64_t d,
                              int64_t B, double* repr) {
  if (!k || !repr || bh < 1 || n < 1 || d < 1 || B < 1) return -1;
  const int64_t nb = ceil_div(n, B);
#pragma omp parallel for schedule(static)
  for (int64_t hb = 0; hb < bh * nb; ++hb) {
    const int64_t h = hb / nb, beta = hb % nb;
    const int64_t j0 = beta * B;
    const int64_t j1 = (j0 + B < n) ? j0 + B : n;
    double* r = repr + hb * d;
    for (int64_t c = 0; c < d; ++c) r[c] = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
      const float* kj = k + (h * n + j) * d;
      for (int64_t c = 0; c < d; ++c) r[c] += (double)kj[c];
    }
    const double cnt = (double)(j1 - j0);
    for (int64_t c = 0; c < d; ++c) r[c] /= cnt;
  }
  return 0;
}

/* Stage 1, coarse scores [P1 "Two-stage block indexer"]: the dot product of
 * the query with every block representative (reading R1: unscaled).
 * scores[r][beta] for each requested row r. */
ORACLE_EXPORT int oracle_scores(const float* q, const double* repr, int64_t bh,
                                int64_t n, int64_t d, int64_t B,
                                const int64_t* rows, int64_t nrows,
                                double* scores) {
  if (!q || !repr || !rows || !scores || bh < 1 || n < 1 || d < 1 || B < 1)
    return -1;
  const int64_t nb = ceil_div(n, B);
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= bh * n) return -2;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t row = rows[r], h = row / n;
    const float* qi = q + row * d;
    for (int64_t beta = 0; beta < nb; ++beta) {
      const double* rb = repr + (h * nb + beta) * d;
      double s = 0.0;
      for (int64_t c = 0; c < d; ++c) s += (double)qi[c] * rb[c];
      scores[r * nb + beta] = s;
    }
  }
  return 0;
}

typedef struct {
  double v;
  int32_t beta;
} cand_t;

/* Descending score, then ascending block index (reading R2).  IEEE comparison
 * makes -0 and +0 compare equal, so they tie and the index decides. */
static int cand_cmp(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->beta > y->beta) - (x->beta < y->beta);
}

static int int_cmp(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Stage 1, selection [P1 "Two-stage block indexer": "take the top-k
 * highest-scoring blocks"], one row at a time.  Candidates are all blocks, or
 * in the causal variant the blocks up to the query's own block, whose score is
 * replaced by +inf so it is always kept (reading R4).  Sort the candidates by
 * (score desc, index asc), keep the first k_eff = min(k, #candidates)
 * (reading R3), emit them in ascending index order, pad with -1.
 * kth[r] / next[r] receive the k_eff-th and (k_eff+1)-th candidate scores in
 * that order (NAN when absent); the tie band is judged on them. */
ORACLE_EXPORT int oracle_topk(const double* scores, const int64_t* rows,
                              int64_t nrows, int64_t n, int64_t nb, int64_t B,
                              int64_t topk, int causal, int32_t* idx,
                              double* kth, double* next) {
  if (!scores || !rows || !idx || n < 1 || nb < 1 || B < 1 || topk < 1)
    return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(| : bad)
  for (int64_t r = 0; r < nrows; ++r) {
    cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)nb);
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)topk);
    if (!c || !sel) {
      bad = 1;
      free(c);
      free(sel);
      continue;
    }
    const int64_t i = rows[r] % n;
    const int64_t qb = i / B;
    int64_t nc = 0;
    for (int64_t beta = 0; beta < nb; ++beta) {
      if (causal && beta > qb) break;
      double v = scores[r * nb + beta];
      if (causal && beta == qb) v = INFINITY;
      c[nc].v = v;
      c[nc].beta = (int32_t)beta;
      ++nc;
    }
    qsort(c, (size_t)nc, sizeof(cand_t), cand_cmp);
    const int64_t keff = nc < topk ? nc : topk;
    for (int64_t t = 0; t < keff; ++t) sel[t] = c[t].beta;
    qsort(sel, (size_t)keff, sizeof(int32_t), int_cmp);
    for (int64_t t = 0; t < topk; ++t) idx[r * topk + t] = t < keff ? sel[t] : -1;
    if (kth) kth[r] = keff > 0 ? c[keff - 1].v : NAN;
    if (next) next[r] = nc > keff ? c[keff].v : NAN;
    free(c);
    free(sel);
  }
  return bad ? -3 : 0;
}

/* Softmax attention of one query over an explicit key list, two passes:
 * z_j = scale * q.k_j ; o = sum_j exp(z_j - max z) v_j / sum_j exp(z_j - max z).
 * An empty list gives o = 0 (reading R6). */
static void attend_list(const float* qi, const float* kh, const float* vh,
                        int64_t d, double scale, const int64_t* keys,
                        int64_t nkeys, double* z, double* o) {
  for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
  if (nkeys == 0) return;
  double zmax = -INFINITY;
  for (int64_t t = 0; t < nkeys; ++t) {
    const float* kj = kh + keys[t] * d;
    double s = 0.0;
    for (int64_t c = 0; c < d; ++c) s += (double)qi[c] * (double)kj[c];
    z[t] = scale * s;
    if (z[t] > zmax) zmax = z[t];
  }
  double den = 0.0;
  for (int64_t t = 0; t < nkeys; ++t) {
    const double w = exp(z[t] - zmax);
    den += w;
    const float* vj = vh + keys[t] * d;
    for (int64_t c = 0; c < d; ++c) o[c] += w * (double)vj[c];
  }
  for (int64_t c = 0; c < d; ++c) o[c] /= den;
}

/* Stage 2 [P1 "Two-stage block indexer", "The Triton kernel"]: for each row,
 * the visible keys are the keys of its selected blocks (entries < 0 are
 * padding), restricted to j <= i in the causal variant (reading R4); the
 * output is softmax attention over exactly those keys.  The block order in
 * idx does not matter.  out[r][:] per requested row. */
ORACLE_EXPORT int oracle_attend(const float* q, const float* k, const float* v,
                                int64_t bh, int64_t n, int64_t d, int64_t B,
                                int64_t topk, int causal, double scale,
                                const int32_t* idx, const int64_t* rows,
                                int64_t nrows, double* out) {
  if (!q || !k || !v || !idx || !rows || !out || bh < 1 || n < 1 || d < 1 ||
      B < 1 || topk < 1)
    return -1;
  const int64_t nb = ceil_div(n, B);
  for (int64_t r = 0; r < nrows; ++r) {
    if (rows[r] < 0 || rows[r] >= bh * n) return -2;
    for (int64_t t = 0; t < topk; ++t)
      if (idx[r * topk + t] >= nb) return -2;
  }
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t row = rows[r], h = row / n, i = row % n;
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(topk * B));
    double* z = (double*)malloc(sizeof(double) * (size_t)(topk * B));
    if (!keys || !z) {
      bad = 1;
      free(keys);
      free(z);
      continue;
    }
    int64_t nk = 0;
    for (int64_t t = 0; t < topk; ++t) {
      const int64_t beta = idx[r * topk + t];
      if (beta < 0) continue;
      for (int64_t j = beta * B; j < beta * B + B && j < n; ++j) {
        if (causal && j > i) continue;
        keys[nk++] = j;
      }
    }
    attend_list(q + row * d, k + h * n * d, v + h * n * d, d, scale, keys, nk,
                z, out + r * d);
    free(keys);
    free(z);
  }
  return bad ? -3 : 0;
}

/* The static pattern of [P2]: mask[i][j] = 1 iff |i - j| <= window or
 * j mod stride == 0 (global keys only; no global queries). */
ORACLE_EXPORT int oracle_window_stride_mask(int64_t n, int64_t window,
                                            int64_t stride, uint8_t* mask) {
  if (!mask || n < 1 || window < 0 || stride < 1) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < n; ++j) {
      const int64_t dist = i > j ? i - j : j - i;
      mask[i * n + j] = (uint8_t)((dist <= window) || (j % stride == 0));
    }
  return 0;
}

/* Masked softmax attention [P2; P3 "Block-Sparse Attention"]: row i sees
 * exactly the keys j with mask[i][j] != 0 (the same mask for every head);
 * masked keys take no part, i.e. they score -inf. */
ORACLE_EXPORT int oracle_attend_mask(const float* q, const float* k,
                                     const float* v, int64_t bh, int64_t n,
                                     int64_t d, double scale,
                                     const uint8_t* mask, const int64_t* rows,
                                     int64_t nrows, double* out) {
  if (!q || !k || !v || !mask || !rows || !out || bh < 1 || n < 1 || d < 1)
    return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= bh * n) return -2;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t row = rows[r], h = row / n, i = row % n;
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    double* z = (double*)malloc(sizeof(double) * (size_t)n);
    if (!keys || !z) {
      bad = 1;
      free(keys);
      free(z);
      continue;
    }
    int64_t nk = 0;
    for (int64_t j = 0; j < n; ++j)
      if (mask[i * n + j]) keys[nk++] = j;
    attend_list(q + row * d, k + h * n * d, v + h * n * d, d, scale, keys, nk,
                z, out + r * d);
    free(keys);
    free(z);
  }
  return bad ? -3 : 0;
}

/* Number of (query, key) pairs the fine stage visits for the given rows and
 * selections: the FLOP count of the fine stage is 4*d times this number
 * (QK^T and PV, one multiply-add each per pair and dimension). */
ORACLE_EXPORT int64_t oracle_visible_pairs(const int32_t* idx,
                                           const int64_t* rows, int64_t nrows,
                                           int64_t n, int64_t B, int64_t topk,
                                           int causal) {
  if (!idx || !rows || n < 1 || B < 1 || topk < 1) return -1;
  int64_t total = 0;
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t i = rows[r] % n;
    for (int64_t t = 0; t < topk; ++t) {
      const int64_t beta = idx[r * topk + t];
      if (beta < 0) continue;
      for (int64_t j = beta * B; j < beta * B + B && j < n; ++j)
        if (!causal || j <= i) ++total;
    }
  }
  return total;
}

/* ------------------------------------------------------------------------
 * Backward of the fine stage [P1 "What's next": a backward pass that
 * differentiates through the softmax-weighted sum over the selected blocks,
 * with FlashAttention-2's backward as the dense model].
 *
 * Reading R7: the selection is a discrete choice and carries no gradient; it
 * is held fixed (the idx the forward used), so the gradients are those of
 * softmax attention over each row's visible key set J(i).  With
 * z_ij = scale * q_i.k_j, p_ij = softmax_j(z_ij) over J(i) and an incoming
 * gradient dO_i of o_i = sum_j p_ij v_j:
 *   dp_ij = dO_i . v_j
 *   ds_ij = p_ij (dp_ij - sum_l p_il dp_il)      (softmax Jacobian)
 *   dq_i  = scale * sum_j ds_ij k_j
 *   dk_j  = scale * sum_{i : j in J(i)} ds_ij q_i
 *   dv_j  = sum_{i : j in J(i)} p_ij dO_i
 * and lse_i = log sum_{j in J(i)} exp(z_ij) (natural log, scale included).
 * ------------------------------------------------------------------------ */

/* Visible keys of row i of one head: the keys of its selected blocks
 * (entries < 0 are padding), j <= i if causal (R4).  Returns the count. */
static int64_t row_keys(const int32_t* sel, int64_t topk, int64_t i, int64_t n,
                        int64_t B, int causal, int64_t* keys) {
  int64_t nk = 0;
  for (int64_t t = 0; t < topk; ++t) {
    const int64_t beta = sel[t];
    if (beta < 0) continue;
    for (int64_t j = beta * B; j < beta * B + B && j < n; ++j) {
      if (causal && j > i) continue;
      keys[nk++] = j;
    }
  }
  return nk;
}

/* Softmax of one row over its key list: p[t] for keys[t], the row's lse,
 * and delta = sum_t p[t] (dO . v_keys[t]).  An empty list gives lse = -inf,
 * delta = 0 (R6). */
static void row_softmax(const float* qi, const float* dOi, const float* kh,
                        const float* vh, int64_t d, double scale,
                        const int64_t* keys, int64_t nk, double* p,
                        double* lse, double* delta) {
  *lse = -INFINITY;
  *delta = 0.0;
  if (nk == 0) return;
  double zmax = -INFINITY;
  for (int64_t t = 0; t < nk; ++t) {
    const float* kj = kh + keys[t] * d;
    double s = 0.0;
    for (int64_t c = 0; c < d; ++c) s += (double)qi[c] * (double)kj[c];
    p[t] = scale * s;
    if (p[t] > zmax) zmax = p[t];
  }
  double den = 0.0;
  for (int64_t t = 0; t < nk; ++t) {
    p[t] = exp(p[t] - zmax);
    den += p[t];
  }
  for (int64_t t = 0; t < nk; ++t) p[t] /= den;
  *lse = zmax + log(den);
  double dl = 0.0;
  for (int64_t t = 0; t < nk; ++t) {
    const float* vj = vh + keys[t] * d;
    double dp = 0.0;
    for (int64_t c = 0; c < d; ++c) dp += (double)dOi[c] * (double)vj[c];
    dl += p[t] * dp;
  }
  *delta = dl;
}

/* Gradients for the requested query rows (dq, lse) and the requested key
 * blocks (dk, dv: kblocks[b] = head * nb + beta, rows of the block past n are
 * zero).  idx holds the selections of ALL bh*n rows ([bh*n][topk]): a key's
 * gradient sums over every row that sees it. */
ORACLE_EXPORT int oracle_attend_backward(
    const float* q, const float* k, const float* v, const float* dout,
    int64_t bh, int64_t n, int64_t d, int64_t B, int64_t topk, int causal,
    double scale, const int32_t* idx, const int64_t* rows, int64_t nrows,
    double* dq, double* lse, const int64_t* kblocks, int64_t nkb, double* dk,
    double* dv) {
  if (!q || !k || !v || !dout || !idx || bh < 1 || n < 1 || d < 1 || B < 1 ||
      topk < 1 || (nrows > 0 && (!rows || !dq || !lse)) ||
      (nkb > 0 && (!kblocks || !dk || !dv)))
    return -1;
  const int64_t nb = ceil_div(n, B);
  for (int64_t r = 0; r < bh * n * topk; ++r)
    if (idx[r] >= nb) return -2;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= bh * n) return -2;
  for (int64_t b = 0; b < nkb; ++b)
    if (kblocks[b] < 0 || kblocks[b] >= bh * nb) return -2;
  int bad = 0;

  /* dq and lse, one row at a time. */
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t row = rows[r], h = row / n, i = row % n;
    const float* kh = k + h * n * d;
    const float* vh = v + h * n * d;
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(topk * B));
    double* p = (double*)malloc(sizeof(double) * (size_t)(topk * B));
    if (!keys || !p) {
      bad = 1;
      free(keys);
      free(p);
      continue;
    }
    const int64_t nk = row_keys(idx + row * topk, topk, i, n, B, causal, keys);
    double delta;
    row_softmax(q + row * d, dout + row * d, kh, vh, d, scale, keys, nk, p,
                &lse[r], &delta);
    double* g = dq + r * d;
    for (int64_t c = 0; c < d; ++c) g[c] = 0.0;
    for (int64_t t = 0; t < nk; ++t) {
      const float* vj = vh + keys[t] * d;
      const float* kj = kh + keys[t] * d;
      double dp = 0.0;
      for (int64_t c = 0; c < d; ++c) dp += (double)dout[row * d + c] * (double)vj[c];
      const double ds = p[t] * (dp - delta);
      for (int64_t c = 0; c < d; ++c) g[c] += scale * ds * (double)kj[c];
    }
    free(keys);
    free(p);
  }
  if (bad) return -3;

  /* dk and dv.  First lse_i and delta_i of every row that selects one of
   * the requested blocks (each over its whole key list); then, one requested
   * block at a time, the sum over the rows of its head in ascending order,
   * with p_ij = exp(z_ij - lse_i). */
  if (nkb == 0) return 0;
  char* want = (char*)calloc((size_t)(bh * n), 1);
  double* rl = (double*)malloc(sizeof(double) * (size_t)(bh * n));
  double* rd = (double*)malloc(sizeof(double) * (size_t)(bh * n));
  if (!want || !rl || !rd) {
    free(want);
    free(rl);
    free(rd);
    return -3;
  }
  for (int64_t b = 0; b < nkb; ++b) {
    const int64_t h = kblocks[b] / nb, beta = kblocks[b] % nb;
    for (int64_t i = 0; i < n; ++i)
      for (int64_t t = 0; t < topk; ++t)
        if (idx[(h * n + i) * topk + t] == beta) want[h * n + i] = 1;
  }
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
  for (int64_t row = 0; row < bh * n; ++row) {
    if (!want[row]) continue;
    const int64_t h = row / n, i = row % n;
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(topk * B));
    double* p = (double*)malloc(sizeof(double) * (size_t)(topk * B));
    if (!keys || !p) {
      bad = 1;
      free(keys);
      free(p);
      continue;
    }
    const int64_t nk = row_keys(idx + row * topk, topk, i, n, B, causal, keys);
    row_softmax(q + row * d, dout + row * d, k + h * n * d, v + h * n * d, d,
                scale, keys, nk, p, &rl[row], &rd[row]);
    free(keys);
    free(p);
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < nkb; ++b) {
    const int64_t h = kblocks[b] / nb, beta = kblocks[b] % nb;
    const float* kh = k + h * n * d;
    const float* vh = v + h * n * d;
    double* gk = dk + b * B * d;
    double* gv = dv + b * B * d;
    for (int64_t e = 0; e < B * d; ++e) gk[e] = gv[e] = 0.0;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t row = h * n + i;
      int64_t hits = 0;
      for (int64_t t = 0; t < topk; ++t) hits += idx[row * topk + t] == beta;
      for (int64_t j = beta * B; j < beta * B + B && j < n; ++j) {
        if (hits == 0 || (causal && j > i)) continue;
        const float* kj = kh + j * d;
        const float* vj = vh + j * d;
        double s = 0.0, dp = 0.0;
        for (int64_t c = 0; c < d; ++c) {
          s += (double)q[row * d + c] * (double)kj[c];
          dp += (double)dout[row * d + c] * (double)vj[c];
        }
        const double pij = exp(scale * s - rl[row]);
        const double ds = pij * (dp - rd[row]);
        /* a block listed twice in a row is two copies of its keys in J(i) */
        for (int64_t c = 0; c < d; ++c) {
          gk[(j - beta * B) * d + c] += (double)hits * scale * ds * (double)q[row * d + c];
          gv[(j - beta * B) * d + c] += (double)hits * pij * (double)dout[row * d + c];
        }
      }
    }
  }
  free(want);
  free(rl);
  free(rd);
  return bad ? -3 : 0;
}
