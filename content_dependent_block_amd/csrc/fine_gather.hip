// fine_gather.hip -- Stage 2 by block-major gathering ("block-gather"):
// every selected (query, block) pair is computed exactly once on MFMA, with
// 16 pairs that share a key block packed into one MFMA tile.
//
// What it computes is the fine stage of nishantmodi.me
// "sparse-attention-triton-bench" (sections "Stage 2: fine attention" and
// "The Triton kernel"): o_i = softmax over the keys of query i's selected
// blocks, applied to V.  Instead of one online-softmax pass per query, the
// softmax is split by block (a standard split-softmax identity): each pair
// (i, beta) yields m = max of its log2-scaled scores, l = sum 2^(z - m),
// o = (sum 2^(z - m) v) / l and its log-sum-exp L = m + log2 l; the pairs of
// a query are then merged as
//   M = max L_s,  w_s = 2^(L_s - M),  o_i = sum w_s o_s / sum w_s.
// No score leaves the chip; only the per-pair rows o do, each carrying its L
// in the least significant bits of its first 32 elements (one 128-byte line
// per pair for bf16 inputs, and no separate record to scatter): for fp16 rows
// the two halves of 32-bit word p (p < 16) carry bits p and p + 16 of L, for
// fp32 rows element e carries bit e.
//
// Why: with content-dependent selections, queries that sit next to each other
// share few blocks, so a query tile's union of blocks is mostly work for one
// or two of its rows.  Grouping pairs by block instead gives full 16-row MFMA
// tiles and reads each K/V block once per 128 pairs.
//
// Kernels, per chunk of query rows (the chunk bounds the partial buffer):
//   bucket_count   -- histogram of the chunk's pairs by (head, query segment,
//                     key block); each pair
//                     gets its rank inside its bucket (LDS histogram per 64 rows,
//                     one global atomic per (workgroup, block)).
//   bucket_scan    -- one workgroup: exclusive prefix of the counts (pair offsets)
//                     and of ceil(count / item_pairs) (work-item offsets).
//   bucket_fill    -- pair ids into per-bucket lists.
//   gather_partial -- one work item = up to 256 pairs of one bucket: K and V^T
//                     of the block in LDS, the pairs' query rows gathered into
//                     MFMA operands, S^T = K Q^T and O^T = V^T P^T on MFMA,
//                     partial rows out.  Work items are laid out so that
//                     consecutive items (one head, one query segment,
//                     neighbouring blocks) land on one XCD, whose L2 then holds
//                     the segment's query rows (at most 4 MB, gather_segments).
//   combine        -- per query row, merge its partials in slot order.
// The order of pairs inside a bucket (set by atomics) does not affect any
// result: every MFMA column is computed independently of the others.
#include <type_traits>

#include "bsa_device.hpp"
#include "bsa_launch.hpp"
#include "kv_tile.hpp"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;

typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Bucket of pair (row, beta): (head, query segment, key block), so that the
// buckets of one segment of one head are consecutive.
__device__ __forceinline__ int64_t bucket_of(int64_t row, int beta, int n, int nb, int qsegs, int64_t bh0) {
  const int seg = static_cast<int>(row % n) / (n / qsegs);
  return ((row / n - bh0) * qsegs + seg) * nb + beta;
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int64_t count) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < count) p[i] = 0;
}

// The candidate blocks of the rows of one bucketing workgroup.  Its rows
// start at r_begin and lie in one slice (rpw divides the segment), so the
// row of its pair e is r_begin + e / topk and its position in the slice
// i0 + e / topk, i0 = r_begin mod n: no 64-bit division per pair, and none
// at all unless a block table or the causal limit needs the row.  e / topk
// comes from a float estimate, which is within one of it for e < 2^22, and
// one correction each way.
struct WgRows {
  int i0, topk, nb, causal;
  float inv_topk;
  const int4* seqtab;
  __device__ __forceinline__ WgRows(int64_t r_begin, int n, int topk_, int causal_, const int4* tab)
      : i0(static_cast<int>(r_begin % n)), topk(topk_), nb(n / kTile), causal(causal_),
        inv_topk(1.0f / static_cast<float>(topk_)), seqtab(tab) {}
  __device__ __forceinline__ RowBlocks of(int e, bool use_causal) const {
    RowBlocks r;
    r.lo = 0;
    r.hi = nb;
    r.own = 0;
    if (seqtab || (use_causal && causal)) {
      int q = static_cast<int>(static_cast<float>(e) * inv_topk);
      q += (q + 1) * topk <= e ? 1 : 0;
      q -= q * topk > e ? 1 : 0;
      r.own = (i0 + q) / kTile;
      if (seqtab) {
        const int4 t = seqtab[r.own];
        r.lo = t.x;
        r.hi = t.y;
      }
      if (use_causal && causal) r.hi = r.own + 1;
    }
    return r;
  }
};

// Pairs per thread the bucketing kernels keep in registers: a workgroup of
// rpw rows holds rpw * topk <= 256 * kPairRegs pairs that way (all the
// selection sizes up to 32 at rpw = 256); larger ones go through memory.
constexpr int kPairRegs = 32;

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Exclusive prefix sum, in place, of s[0 .. m) in LDS (m <= 2048) by a
// 256-thread workgroup; returns the total.  wt: 4 ints of LDS.
__device__ __forceinline__ int32_t block_excl_scan(int32_t* s, int m, int32_t* wt) {
  constexpr int P = 8;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int32_t v[P], sum = 0;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    v[j] = t * P + j < m ? s[t * P + j] : 0;
    sum += v[j];
  }
  const int32_t inc = wave_incl_scan(sum, lane);
  if (lane == 63) wt[wave] = inc;
  __syncthreads();
  int32_t run = inc - sum, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) run += wt[w];
    total += wt[w];
  }
#pragma unroll
  for (int j = 0; j < P; ++j) {
    if (t * P + j < m) s[t * P + j] = run;
    run += v[j];
  }
  __syncthreads();
  return total;
}

// One workgroup per `rpw` query rows of one query segment (rpw divides the
// segment length and row0).  Each pair's rank inside its bucket is its
// workgroup's base (one global atomic per (workgroup, block)) plus its rank
// inside the workgroup (LDS atomics).
//
// Register path (rpw * topk <= 256 * kPairRegs): the workgroup's valid pairs
// also leave ordered by block, as records {pair, block << 21 | rank} at
// rec[first pair of the workgroup + position], with the count of valid pairs
// in wg_valid[workgroup] (a bucket holds pairs of distinct rows of one head,
// so rank < n <= 2^17 fits 21 bits and the block 11).  Otherwise each pair's
// rank goes to rank[pair] (-1 for padding).
__global__ __launch_bounds__(256) void bucket_count_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ count, int32_t* __restrict__ rank,
    int2* __restrict__ rec, int32_t* __restrict__ wg_valid, int64_t row0, int64_t rows, int n, int topk,
    int causal, int64_t bh0, int rpw, int qsegs, const int4* __restrict__ seqtab) {
  // LDS: [nb] local counts -> local offsets, [nb] global bases, [4] scan
  // scratch, then (register path) the block-ordered records, 8 bytes each
  extern __shared__ int32_t hist[];
  const int nb = n / kTile;
  int32_t* base = hist + nb;
  const int64_t r_begin = row0 + static_cast<int64_t>(blockIdx.x) * rpw;
  const int64_t nrows = (row0 + rows - r_begin) < rpw ? (row0 + rows - r_begin) : rpw;
  const int npairs = static_cast<int>(nrows) * topk;
  const int64_t p_begin = (r_begin - row0) * topk;  // chunk-relative pair id of the first pair
  const int64_t bucket0 = bucket_of(r_begin, 0, n, nb, qsegs, bh0);  // rpw divides the segment
  const int32_t* sel = idx + r_begin * topk;          // the workgroup's selections, contiguous
  const WgRows wr(r_begin, n, topk, causal, seqtab);
  for (int c = threadIdx.x; c < nb; c += 256) hist[c] = 0;
  __syncthreads();
  if (npairs <= 256 * kPairRegs) {
    int32_t lr[kPairRegs], bt[kPairRegs];
#pragma unroll
    for (int j = 0; j < kPairRegs; ++j) {
      const int e = threadIdx.x + 256 * j;
      lr[j] = -1;
      bt[j] = 0;
      if (e < npairs) {
        const int beta = sel_block(sel[e], wr.of(e, true));
        if (beta >= 0) {
          bt[j] = beta;
          lr[j] = atomicAdd(&hist[beta], 1);
        }
      }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < nb; c += 256)
      base[c] = hist[c] ? atomicAdd(&count[bucket0 + c], hist[c]) : 0;
    __syncthreads();
    const int32_t valid = block_excl_scan(hist, nb, hist + 2 * nb);
    if (threadIdx.x == 0) wg_valid[blockIdx.x] = valid;
    // ordered in LDS, then written out contiguously
    int2* srec = reinterpret_cast<int2*>(hist + 2 * nb + 4);
#pragma unroll
    for (int j = 0; j < kPairRegs; ++j) {
      const int e = threadIdx.x + 256 * j;
      if (lr[j] >= 0)
        srec[hist[bt[j]] + lr[j]] =
            make_int2(static_cast<int32_t>(p_begin + e),
                      static_cast<int32_t>((static_cast<uint32_t>(bt[j]) << 21) |
                                           static_cast<uint32_t>(base[bt[j]] + lr[j])));
    }
    __syncthreads();
    for (int t = threadIdx.x; t < valid; t += 256) rec[p_begin + t] = srec[t];
    return;
  }
  for (int e = threadIdx.x; e < npairs; e += 256) {
    const int beta = sel_block(sel[e], wr.of(e, true));
    rank[p_begin + e] = beta >= 0 ? atomicAdd(&hist[beta], 1) : -1;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < nb; c += 256)
    base[c] = hist[c] ? atomicAdd(&count[bucket0 + c], hist[c]) : 0;
  __syncthreads();
  for (int e = threadIdx.x; e < npairs; e += 256) {
    const int32_t rk = rank[p_begin + e];
    if (rk >= 0) rank[p_begin + e] = base[sel_block(sel[e], wr.of(e, false))] + rk;
  }
}

// The bucket scan (bucket_scan_kernel, below, states what it computes) for
// up to 4096 buckets, in one step: thread t takes buckets 4t .. 4t + 3
// (loaded, summed, scanned over the workgroup through the 16 wave totals,
// written back and cleared), with no LDS staging and no passes.
constexpr int kScanSmallMax = 4096;
__global__ __launch_bounds__(1024) void bucket_scan_small_kernel(int32_t* __restrict__ count,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ items, int nbuckets,
                                                                 int item_pairs) {
  __shared__ int32_t s_wp[16], s_wi[16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int32_t v[4], sp = 0, si = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 4 * t + j;
    v[j] = b < nbuckets ? count[b] : 0;
    sp += v[j];
    si += (v[j] + item_pairs - 1) / item_pairs;
  }
  const int32_t ip = wave_incl_scan(sp, lane), ii = wave_incl_scan(si, lane);
  if (lane == 63) {
    s_wp[wave] = ip;
    s_wi[wave] = ii;
  }
  __syncthreads();
  int32_t ep = ip - sp, ei = ii - si, tp = 0, ti = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    if (w < wave) {
      ep += s_wp[w];
      ei += s_wi[w];
    }
    tp += s_wp[w];
    ti += s_wi[w];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 4 * t + j;
    if (b < nbuckets) {
      offsets[b] = ep;
      items[b] = ei;
      count[b] = 0;  // the counts start at zero for the next bucketing
    }
    ep += v[j];
    ei += (v[j] + item_pairs - 1) / item_pairs;
  }
  if (t == 0) {
    offsets[nbuckets] = tp;
    items[nbuckets] = ti;
  }
}

// Single workgroup of 1024 threads.  offsets[b] / items[b] are exclusive
// prefixes; entry nbuckets holds the totals.  It leaves count[] zero, as the
// next bucketing's count kernel needs it.  Passes of 1024 x 16 buckets:
// the counts are loaded coalesced into LDS, each thread sums a contiguous run
// of 16, one block-wide scan of the run sums (waves, then the 16 wave totals)
// gives every run its base, and the prefixes go back through LDS to
// coalesced stores.  Runs are padded to 17 words (no bank conflicts).
constexpr int kScanRun = 16;
__global__ __launch_bounds__(1024) void bucket_scan_kernel(int32_t* __restrict__ count,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ items,
                                                           int nbuckets, int item_pairs) {
  constexpr int PASS = 1024 * kScanRun, RP = kScanRun + 1;
  __shared__ int32_t s_c[1024 * RP], s_i[1024 * RP];
  __shared__ int32_t s_wp[16], s_wi[16], s_tot[2];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int32_t carry_p = 0, carry_i = 0;
  for (int base = 0; base < nbuckets; base += PASS) {
#pragma unroll
    for (int j = 0; j < kScanRun; ++j) {
      const int e = j * 1024 + t, b = base + e;  // element e of the pass lives in run e / 16
      s_c[(e / kScanRun) * RP + e % kScanRun] = b < nbuckets ? count[b] : 0;
      if (b < nbuckets) count[b] = 0;  // the counts start at zero for the next bucketing
    }
    __syncthreads();
    int32_t v[kScanRun], sp = 0, si = 0;
#pragma unroll
    for (int j = 0; j < kScanRun; ++j) {
      v[j] = s_c[t * RP + j];
      sp += v[j];
      si += (v[j] + item_pairs - 1) / item_pairs;
    }
    const int32_t ip = wave_incl_scan(sp, lane), ii = wave_incl_scan(si, lane);
    if (lane == 63) {
      s_wp[wave] = ip;
      s_wi[wave] = ii;
    }
    __syncthreads();
    if (wave == 0) {
      const int32_t wp = lane < 16 ? s_wp[lane] : 0, wi = lane < 16 ? s_wi[lane] : 0;
      const int32_t xp = wave_incl_scan(wp, lane), xi = wave_incl_scan(wi, lane);
      if (lane < 16) {
        s_wp[lane] = xp - wp;
        s_wi[lane] = xi - wi;
      }
      if (lane == 15) {
        s_tot[0] = xp;
        s_tot[1] = xi;
      }
    }
    __syncthreads();
    int32_t ep = carry_p + s_wp[wave] + ip - sp, ei = carry_i + s_wi[wave] + ii - si;
#pragma unroll
    for (int j = 0; j < kScanRun; ++j) {
      s_c[t * RP + j] = ep;
      s_i[t * RP + j] = ei;
      ep += v[j];
      ei += (v[j] + item_pairs - 1) / item_pairs;
    }
    carry_p += s_tot[0];
    carry_i += s_tot[1];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kScanRun; ++j) {
      const int e = j * 1024 + t, b = base + e;
      if (b < nbuckets) {
        offsets[b] = s_c[(e / kScanRun) * RP + e % kScanRun];
        items[b] = s_i[(e / kScanRun) * RP + e % kScanRun];
      }
    }
    __syncthreads();
  }
  if (t == 0) {
    offsets[nbuckets] = carry_p;
    items[nbuckets] = carry_i;
  }
}

// Pair ids into per-bucket lists, with the geometry of bucket_count (one
// workgroup per rpw rows).  On the register path it streams the count
// kernel's block-ordered records, so the pairs of one bucket, whose list
// positions are consecutive, leave in consecutive lanes of one store; else
// each pair is stored at its own position.  The list starts of the
// workgroup's (head, segment) are staged in LDS first when they fit
// (stage_off, nb entries), and a thread issues the loads of all its records
// before storing any, so a record costs one global load rather than a chain
// of two.  Workgroup w also
// writes, for each work item of buckets 256w .. 256w + 255, the record
// {bucket, first list position, pair count} at the slot of the workgroup
// that will run it: items are spread so that consecutive items (one head,
// neighbouring blocks) go to one XCD, i.e. item = xcd * per_xcd + j runs as
// workgroup j * 8 + xcd.
__global__ __launch_bounds__(256) void bucket_fill_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ rank, const int2* __restrict__ rec,
    const int32_t* __restrict__ wg_valid, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ items, int4* __restrict__ item_rec, int nbuckets, int64_t max_slots,
    int32_t* __restrict__ list, int64_t row0, int64_t rows, int n, int topk, int64_t bh0, int qsegs,
    int item_pairs, int rpw, const int4* __restrict__ seqtab, int stage_off) {
  extern __shared__ int32_t s_off[];  // [nb] when stage_off
  const int64_t pb = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (pb < nbuckets) {
    const int32_t total = items[nbuckets];
    const int32_t per_xcd = (total + kXcds - 1) / kXcds;
    const int32_t cnt = offsets[pb + 1] - offsets[pb];
    for (int32_t i = items[pb], u = 0; i < items[pb + 1]; ++i, ++u) {
      const int64_t slot = static_cast<int64_t>(i % per_xcd) * kXcds + i / per_xcd;
      const int32_t left = cnt - u * item_pairs;
      if (slot < max_slots)
        item_rec[slot] = make_int4(static_cast<int32_t>(pb), offsets[pb] + u * item_pairs,
                                   left < item_pairs ? left : item_pairs, 0);
    }
  }
  const int64_t r_begin = row0 + static_cast<int64_t>(blockIdx.x) * rpw;
  if (r_begin >= row0 + rows) return;  // workgroup-uniform: no rows here
  const int nb = n / kTile;
  const int64_t nrows = (row0 + rows - r_begin) < rpw ? (row0 + rows - r_begin) : rpw;
  const int np = static_cast<int>(nrows) * topk;
  const int64_t npairs = rows * topk;
  const int64_t p_begin = (r_begin - row0) * topk;
  const int32_t* off = offsets + bucket_of(r_begin, 0, n, nb, qsegs, bh0);  // rpw divides the segment
  if (np <= 256 * kPairRegs) {
    // the count kernel's block-ordered records: consecutive records of one
    // block have consecutive list positions
    const int32_t valid = wg_valid[blockIdx.x];
    if (stage_off) {  // workgroup-uniform
      for (int c = threadIdx.x; c < nb; c += 256) s_off[c] = off[c];
      __syncthreads();
      int2 r[kPairRegs];
#pragma unroll
      for (int j = 0; j < kPairRegs; ++j) {
        const int t = threadIdx.x + 256 * j;
        r[j] = t < valid ? rec[p_begin + t] : make_int2(0, -1);
      }
#pragma unroll
      for (int j = 0; j < kPairRegs; ++j) {
        const int t = threadIdx.x + 256 * j;
        const uint32_t w = static_cast<uint32_t>(r[j].y);
        if (t < valid) {
          const int64_t pos = static_cast<int64_t>(s_off[w >> 21]) + (w & 0x1FFFFFu);
          if (pos < npairs) list[pos] = r[j].x;
        }
      }
      return;
    }
    for (int t = threadIdx.x; t < valid; t += 256) {
      const int2 r = rec[p_begin + t];
      const uint32_t w = static_cast<uint32_t>(r.y);
      const int64_t pos = static_cast<int64_t>(off[w >> 21]) + (w & 0x1FFFFFu);
      if (pos < npairs) list[pos] = r.x;
    }
    return;
  }
  const int32_t* sel = idx + r_begin * topk;
  const WgRows wr(r_begin, n, topk, 0, seqtab);
  for (int e = threadIdx.x; e < np; e += 256) {
    const int32_t rk = rank[p_begin + e];
    if (rk < 0) continue;
    const int64_t pos = static_cast<int64_t>(off[sel_block(sel[e], wr.of(e, false))]) + rk;
    if (pos < npairs) list[pos] = static_cast<int32_t>(p_begin + e);
  }
}

// bf16 inputs keep partial outputs as fp16, fp32 inputs as fp32.  An fp16
// row (|o| <= max |v|) is rounded once (half an ulp) and its first 32
// elements lose their last mantissa bit to the log-sum-exp (up to one ulp
// more): at most 1.5 ulp, 1.5 * 2^-10 relative, so an absolute error of up
// to 1.5 * 2^-10 * max |v| per element.
template <typename T>
using PartialT = typename std::conditional<sizeof(T) == 2, f16, float>::type;

// Query operand of S^T = K Q^T for one lane: its pair's query row, the d
// slots of MFMA k-group lane/16.
template <typename T, int D>
union QOperand {
  bf16x8 b[D / 32];
  float f[D / 4];
};

template <typename T, int D>
__device__ __forceinline__ void load_q(QOperand<T, D>& qo, const T* __restrict__ q, int64_t row,
                                       bool live, int g) {
  if constexpr (sizeof(T) == 2) {
    const T* qp = q + row * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qo.b[kk] = live ? as_bf16x8(ld16(qp + 32 * kk)) : bf16x8{};
  } else {
    constexpr int KS = D / 4;
    const T* qp = q + row * D + KS * g;
#pragma unroll
    for (int e = 0; e < KS; e += 4) {
      const uint4 u = live ? ld16(qp + e) : uint4{0u, 0u, 0u, 0u};
      qo.f[e] = __uint_as_float(u.x);
      qo.f[e + 1] = __uint_as_float(u.y);
      qo.f[e + 2] = __uint_as_float(u.z);
      qo.f[e + 3] = __uint_as_float(u.w);
    }
  }
}

// Row pitch (fp16 elements) of a wave's LDS staging rows for the partial
// outputs: 16 bytes of padding between rows.
template <int D>
constexpr int kStagePitch = D + 8;

// Output dim carried by row m of PV output tile dt (bf16 path).  The V^T
// rows fed to each MFMA tile are permuted so that the lanes of row group
// g = m/4 end up holding 8 consecutive dims per pair of tiles: tiles 2u and
// 2u+1 cover dims 32u .. 32u+31, group g takes 32u + 8g .. 32u + 8g + 7, the
// first tile of the pair the lower 4 of those.  A bijection on 0 .. D-1.
template <int D>
__device__ __forceinline__ int out_dim(int dt, int m) {
  return 32 * (dt / 2) + 8 * (m / 4) + 4 * (dt % 2) + (m % 4);
}

// One group of 16 pairs sharing key block `beta` (K, V^T in LDS): the lane
// computes column lane%16 (its pair) and writes the pair's partial row
// o = sum 2^(z-m) v / l with m + log2 l in its low bits (m in log2 units,
// l = sum 2^(z-m)).  The softmax scale is folded
// into the exp2 argument (the max is taken on raw scores; the scale is > 0),
// and for bf16 inputs l comes out of the PV MFMA itself: one more output
// tile whose A operand is all ones multiplies the same rounded
// probabilities, so l sums exactly the weights that enter o, and every row
// of that tile, hence every lane of the pair's column, holds it.
template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void pair_group(const T* ks, const T* vs, f16* stage, const QOperand<T, D>& qo,
                                           int qi, int beta, int klim, bool live, int32_t pair,
                                           float scale_log2, PartialT<T>* __restrict__ po, int lane) {
  using L = KvLayout<T, D>;
  const int g = lane >> 4, c16 = lane & 15;
  f32x4 s[4];
  if constexpr (L::kBf16) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (16 * tt + c16) * L::KPITCH + 8 * g + 32 * kk);
        s[tt] = mfma_16x16x32_bf16(a, qo.b[kk], s[tt]);
      }
    }
  } else {
    constexpr int KS = D / 4;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const T* kr = ks + (16 * tt + c16) * L::KPITCH + KS * g;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) s[tt] = mfma_16x16x4_f32(kr[kk], qo.f[kk], s[tt]);
    }
  }
  if (CAUSAL) {
    if (beta == qi / kTile) {  // diagonal block: keys after the query are hidden
      const int qlocal = qi % kTile;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (16 * tt + 4 * g + jj > qlocal) s[tt][jj] = -INFINITY;
    }
  }
  if (klim < kTile) {  // a partial last block: keys klim .. 63 are padding
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        if (16 * tt + 4 * g + jj >= klim) s[tt][jj] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
    mx = fmaxf(mx, fmaxf(fmaxf(s[tt][0], s[tt][1]), fmaxf(s[tt][2], s[tt][3])));
  mx = max_over_groups(mx);         // a live pair has >= 1 visible key: finite
  const float m = mx * scale_log2;  // log2-domain max
  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lt;
  if constexpr (L::kBf16) {
    bf16x8 bp[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bp[kk][i] = f32_to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * kk][i], scale_log2, -m)));
        bp[kk][4 + i] = f32_to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * kk + 1][i], scale_log2, -m)));
      }
    const __bf16 one = static_cast<__bf16>(1.0f);
    const bf16x8 ones = {one, one, one, one, one, one, one, one};
    f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const T* vr = vs + out_dim<D>(dt, c16) * L::VPITCH + 32 * kk + 4 * g;
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + 16);
        const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[dt] = mfma_16x16x32_bf16(a, bp[kk], acc[dt]);
      }
      lacc = mfma_16x16x32_bf16(ones, bp[kk], lacc);
    }
    lt = lacc[0];  // C[m][c16] = l of pair c16 for every row m
  } else {
    float p[4][4];
    float lsum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        p[tt][jj] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][jj], scale_log2, -m));
        lsum += p[tt][jj];
      }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const T* vr = vs + (16 * tt + 4 * g + jj) * L::VPITCH + c16;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) acc[dt] = mfma_16x16x4_f32(vr[16 * dt], p[tt][jj], acc[dt]);
      }
    lt = sum_over_groups(lsum);
  }
  // l >= 1 (the maximum's own weight is 1): the hardware reciprocal (1 ulp)
  // is far inside the fp16 rounding of the row it scales.
  const float inv = __builtin_amdgcn_rcpf(lt);
  // The pair's log2-domain log-sum-exp, m + log2 l, rides in the row itself.
  const uint32_t lse_bits = __float_as_uint(m + __builtin_amdgcn_logf(lt));
  if constexpr (L::kBf16) {
    // Through the wave's LDS staging rows (16 pairs x D fp16) so that every
    // partial row leaves as whole 128-byte lines: CPR lanes write one row's
    // CPR 16-byte chunks in one instruction.  Non-temporal stores: the rows
    // are read back only by the combine, and keeping them out of L2 leaves
    // it to the gathered query rows.
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      const f32x4 a0 = acc[2 * u] * inv, a1 = acc[2 * u + 1] * inv;
      const f16x8 h = {static_cast<f16>(a0[0]), static_cast<f16>(a0[1]), static_cast<f16>(a0[2]),
                       static_cast<f16>(a0[3]), static_cast<f16>(a1[0]), static_cast<f16>(a1[1]),
                       static_cast<f16>(a1[2]), static_cast<f16>(a1[3])};
      u32x4 w = __builtin_bit_cast(u32x4, h);
      if (u == 0) {
        // The lane holds elements 8 g .. 8 g + 7, i.e. 32-bit words 4 g + j of
        // the row; word p takes bits p and p + 16 of the log-sum-exp in the
        // least significant bits of its two halves.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t t = lse_bits >> (4 * g + j);
          w[j] = (t & 0x00010001u) | (w[j] & 0xFFFEFFFEu);
        }
      }
      *reinterpret_cast<u32x4*>(stage + c16 * kStagePitch<D> + out_dim<D>(2 * u, 4 * g)) = w;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int CPR = D * 2 / 16;  // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;    // rows per store instruction
    const int32_t pl = live ? pair : -1;  // the row's pair, or -1 for a dead row
#pragma unroll
    for (int i = 0; i < 16 / RPI; ++i) {
      const int r = i * RPI + lane / CPR, ch = lane % CPR;
      const int32_t pr = __shfl(pl, r);
      const u32x4 h = *reinterpret_cast<const u32x4*>(stage + r * kStagePitch<D> + ch * 8);
      if (pr >= 0) __builtin_nontemporal_store(h, reinterpret_cast<u32x4*>(po + static_cast<int64_t>(pr) * D) + ch);
    }
  } else {
    if (!live) return;
    PartialT<T>* op = po + static_cast<int64_t>(pair) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const f32x4 a = acc[dt] * inv;
      uint32_t u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 16 * dt + 4 * g + i;  // element of the row
        u[i] = __float_as_uint(a[i]);
        if (e < 32) u[i] = (u[i] & ~1u) | ((lse_bits >> e) & 1u);
      }
      *reinterpret_cast<uint4*>(op + 16 * dt + 4 * g) = make_uint4(u[0], u[1], u[2], u[3]);
    }
  }
}

// Query operands in flight ahead of the 16-pair group being computed: two
// keeps the d = 64 kernel at 88 VGPRs (5 waves per SIMD; all eight groups'
// rows at once took 120 VGPRs, 4 waves) and was faster than three or four.
constexpr int kQueryAhead = 2;

// One work item = up to IP pairs of one bucket (head, key block),
// described by the record the fill kernel left at this workgroup's slot.
// The loads the item needs are issued before the first is waited on: the
// wave's list entries, the block's K/V into registers, and the query rows of
// its first kQueryAhead groups; then K/V go to LDS and the MFMA work runs,
// each group issuing the query rows of the group kQueryAhead after it.
// row = pair / topk uses a precomputed multiply-shift (exact for pair < 2^31).
template <typename T, int D, bool CAUSAL, int IP>
__global__ __launch_bounds__(256) void gather_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ list, const int32_t* __restrict__ items,
    const int4* __restrict__ item_rec, int nbuckets, int64_t row0, int64_t npairs, int n,
    uint64_t div_magic, int div_shift, int64_t bh0, int qsegs, const int4* __restrict__ seqtab,
    float scale_log2, PartialT<T>* __restrict__ po) {
  using L = KvLayout<T, D>;
  constexpr int GPW = IP / 16 / 4;  // 16-pair groups per wave
  constexpr int STAGE_BYTES = L::kBf16 ? 16 * kStagePitch<D> * 2 : 0;  // per wave
  __shared__ __align__(16) unsigned char smem[L::BYTES + 4 * STAGE_BYTES];
  T* ks = reinterpret_cast<T*>(smem);
  T* vs = reinterpret_cast<T*>(smem + L::K_BYTES);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  f16* stage = reinterpret_cast<f16*>(smem + L::BYTES + wave * STAGE_BYTES);
  const int g = lane >> 4, c16 = lane & 15;

  const int total = items[nbuckets];
  const int4 rec = item_rec[blockIdx.x];
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int slot = static_cast<int>(blockIdx.x) / kXcds;
  const int item = (static_cast<int>(blockIdx.x) % kXcds) * per_xcd + slot;
  if (slot >= per_xcd || item >= total) return;  // no item for this workgroup
  const int b = rec.x;
  if (b < 0 || b >= nbuckets) return;
  const int64_t first = rec.y;
  int cnt = rec.z;
  if (cnt > IP) cnt = IP;
  if (first + cnt > npairs) cnt = first < npairs ? static_cast<int>(npairs - first) : 0;
  const int nb = n / kTile;
  const int beta = b % nb;
  const int64_t bh = bh0 + b / (nb * qsegs);
  const int klim = block_keys(seqtab, beta);  // keys of the block that exist

  int32_t pair[GPW];
  bool live[GPW];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int t = (wave + 4 * gi) * 16 + c16;
    live[gi] = t < cnt;
    pair[gi] = live[gi] ? list[first + t] : 0;
  }
  KvRegs<T, D> kv;
  kv_load<T, D>(kv, k + bh * static_cast<int64_t>(n) * D, v + bh * static_cast<int64_t>(n) * D,
                beta, tid);
  QOperand<T, D> qo[GPW];
  int64_t row[GPW];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    if (pair[gi] < 0 || pair[gi] >= npairs) {
      pair[gi] = 0;
      live[gi] = false;
    }
    row[gi] = row0 + static_cast<int64_t>((static_cast<uint64_t>(pair[gi]) * div_magic) >> div_shift);
    if (gi < kQueryAhead) load_q<T, D>(qo[gi], q, row[gi], live[gi], g);
  }
  kv_store<T, D>(kv, ks, vs, tid);
  __syncthreads();
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    if ((wave + 4 * gi) * 16 >= cnt) break;  // wave-uniform
    if (gi + kQueryAhead < GPW)
      load_q<T, D>(qo[gi + kQueryAhead], q, row[gi + kQueryAhead], live[gi + kQueryAhead], g);
    // the pair's row within its slice: a bucket holds rows of head bh only
    pair_group<T, D, CAUSAL>(ks, vs, stage, qo[gi], static_cast<int>(row[gi] - bh * n), beta, klim, live[gi],
                             pair[gi], scale_log2, po, lane);
  }
}

// Reduce-scatter by OR over a group of 16 lanes: lane c holds v[t] for
// t = 0 .. 15 and gets back the OR of every lane's v[c].  Recursive halving:
// at distance M a lane keeps the half of its 2M live entries whose bit M
// matches its own lane bit and sends the other half to lane c ^ M; after the
// steps M = 8, 4, 2, 1 (15 shuffles) entry 0 is the lane's own slot.
template <int M>
__device__ __forceinline__ void or_halve(uint32_t (&v)[16], int c) {
  const bool hi = (c & M) != 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const uint32_t keep = hi ? v[j + M] : v[j];
    const uint32_t give = hi ? v[j] : v[j + M];
    v[j] = keep | static_cast<uint32_t>(__shfl_xor(static_cast<int>(give), M, 16));
  }
}
__device__ __forceinline__ uint32_t or_scatter16(uint32_t (&v)[16], int c) {
  or_halve<8>(v, c);
  or_halve<4>(v, c);
  or_halve<2>(v, c);
  or_halve<1>(v, c);
  return v[0];
}

// One group of 16 lanes per query row, 16 slots at a time: every lane issues
// the loads of its D/16 dims of all 16 partial rows before using any (slot
// index clamped into the row, so every load is in bounds).  Lane c decides
// whether slot s0 + c counts, a ballot shares the 16 answers with the row's
// lanes, and the words of a slot that does not count (its row was never
// written) are zeroed, so the weighted sum needs no select per element.  Each
// row carries its pair's log2-domain log-sum-exp in the low bits of its
// first 32 elements; lane c collects the bits it holds and a reduce-scatter
// hands lane c the value of slot c.  Rows are merged in slot order against a
// running maximum (rescaled when a later batch of 16 raises it).  Any topk.
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ idx,
                                                      const PartialT<T>* __restrict__ po,
                                                      float* __restrict__ out, float* __restrict__ lse,
                                                      int64_t row0, int64_t rows, int n, int topk,
                                                      int causal, const int4* __restrict__ seqtab) {
  constexpr int E = D / 16;                         // dims per lane
  constexpr int LW = E * sizeof(PartialT<T>) / 4;   // 32-bit words per lane and slot
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  const int gbase = (threadIdx.x & 63) & ~15;
  const bool row_ok = r < rows;  // lanes of a missing row still take part in the ballot
  const int64_t rc = row_ok ? r : rows - 1;
  const int64_t row = row0 + rc;
  const RowBlocks rb = row_blocks(seqtab, row, n, causal);
  const int32_t* sel = idx + row * topk;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float wsum = 0.f, mrun = -INFINITY;
  const PartialT<T>* src = po + rc * topk * D + c * E;
  for (int s0 = 0; s0 < topk; s0 += 16) {
    uint32_t w[16][LW];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int st = s0 + t < topk ? s0 + t : topk - 1;
      const PartialT<T>* p = src + static_cast<int64_t>(st) * D;
      if constexpr (LW == 2) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        w[t][0] = v.x;
        w[t][1] = v.y;
      } else {
#pragma unroll
        for (int h = 0; h < LW / 4; ++h) {
          const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + h);
          w[t][4 * h] = v.x;
          w[t][4 * h + 1] = v.y;
          w[t][4 * h + 2] = v.z;
          w[t][4 * h + 3] = v.w;
        }
      }
    }
    const bool valid = row_ok && s0 + c < topk && sel_block(sel[s0 + c], rb) >= 0;
    const uint32_t vmask = static_cast<uint32_t>(ballot(valid) >> gbase) & 0xFFFFu;
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
      for (int k2 = 0; k2 < LW; ++k2) w[t][k2] = ((vmask >> t) & 1u) ? w[t][k2] : 0u;
    // The bits of each slot's log-sum-exp that this lane holds (lanes
    // c < 32 / E).  fp16 rows: its word k is row word p = c E / 2 + k, whose
    // halves carry bits p and p + 16; fp32 rows: element c E + k carries bit
    // c E + k.
    uint32_t part[16];
    if constexpr (sizeof(PartialT<T>) == 2) {
      const uint32_t msk = c * E < 32 ? 0x00010001u : 0u;
      const int sh = c * E / 2;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        uint32_t b = 0u;
#pragma unroll
        for (int k2 = 0; k2 < LW; ++k2) b |= (w[t][k2] & msk) << k2;
        part[t] = b << sh;
      }
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        uint32_t b = 0u;
#pragma unroll
        for (int k2 = 0; k2 < LW; ++k2) b |= (w[t][k2] & 1u) << k2;
        part[t] = c * E < 32 ? b << (c * E) : 0u;
      }
    }
    const uint32_t bits = or_scatter16(part, c);  // slot s0 + c
    const float ls = valid ? __uint_as_float(bits) : -INFINITY;
    float mb = ls;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) mb = fmaxf(mb, __shfl_xor(mb, off, 16));
    const float mnew = fmaxf(mrun, mb);
    if (mnew > mrun && mrun > -INFINITY) {  // a later batch raised the maximum
      const float sc = __builtin_amdgcn_exp2f(mrun - mnew);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] *= sc;
      wsum *= sc;
    }
    mrun = mnew;
    const float wl = valid ? __builtin_amdgcn_exp2f(ls - mrun) : 0.f;  // weight of slot s0 + c
    wsum += wl;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float ws = __shfl(wl, gbase + t);
      if constexpr (sizeof(PartialT<T>) == 2) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int k2 = 0; k2 < LW; ++k2) {
          const h2 hv = __builtin_bit_cast(h2, w[t][k2]);
          acc[2 * k2] = __builtin_fmaf(static_cast<float>(hv[0]), ws, acc[2 * k2]);
          acc[2 * k2 + 1] = __builtin_fmaf(static_cast<float>(hv[1]), ws, acc[2 * k2 + 1]);
        }
      } else {
#pragma unroll
        for (int k2 = 0; k2 < LW; ++k2) acc[k2] = __builtin_fmaf(__uint_as_float(w[t][k2]), ws, acc[k2]);
      }
    }
  }
  if (!row_ok) return;
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off, 16);
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  // log-sum-exp of the row's scaled scores, natural log: the partial values
  // are in log2 units, so lse = (M + log2 sum_s w_s) / log2(e).
  if (lse && c == 0) lse[row] = wsum > 0.f ? (mrun + __log2f(wsum)) * (1.0f / kLog2e) : -INFINITY;
  float* dst = out + row * D + c * E;
#pragma unroll
  for (int e = 0; e < E; e += 4)
    *reinterpret_cast<float4*>(dst + e) =
        make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
}

struct ChunkGeom {
  int nb, nbuckets;
  int64_t bh0, npairs;
  ChunkGeom(const GatherArgs& a, int64_t row0, int64_t rows) {
    nb = a.n / kTile;
    bh0 = row0 / a.n;
    const int64_t bh1 = (row0 + rows - 1) / a.n;
    nbuckets = static_cast<int>((bh1 - bh0 + 1) * a.qsegs * nb);
    npairs = rows * a.topk;
  }
};

template <typename T, int D>
hipError_t partial_chunk(const GatherArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  constexpr int IP = gather_item_pairs(D, std::is_same<T, float>::value ? BSA_FP32 : BSA_BF16);
  if (a.item_pairs != IP) return hipErrorInvalidValue;  // items made for another kernel
  const ChunkGeom c(a, row0, rows);
  const int64_t grid = gather_grid(rows, a.topk, c.nbuckets, IP);
  const float sl2 = a.scale * kLog2e;
  auto* po = reinterpret_cast<PartialT<T>*>(a.ws.partial_o);
  // pair / topk as (pair * magic) >> shift: shift = 32 + ceil(log2 topk),
  // magic = ceil(2^shift / topk); exact for every pair < 2^31.
  int lg = 0;
  while ((1 << lg) < a.topk) ++lg;
  const int shift = 32 + lg;
  const uint64_t magic = ((uint64_t(1) << shift) + uint64_t(a.topk) - 1) / uint64_t(a.topk);
  if (a.causal)
    hipLaunchKernelGGL((gather_partial_kernel<T, D, true, IP>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, s, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.ws.list, a.ws.items, a.ws.item_rec, c.nbuckets,
                       row0, c.npairs, a.n, magic, shift, c.bh0, a.qsegs, a.seqtab, sl2, po);
  else
    hipLaunchKernelGGL((gather_partial_kernel<T, D, false, IP>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, s, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.ws.list, a.ws.items, a.ws.item_rec, c.nbuckets,
                       row0, c.npairs, a.n, magic, shift, c.bh0, a.qsegs, a.seqtab, sl2, po);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t combine_chunk(const GatherArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  auto* po = reinterpret_cast<const PartialT<T>*>(a.ws.partial_o);
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0,
                     s, a.idx, po, a.out, a.lse, row0, rows, a.n, a.topk, a.causal, a.seqtab);
  return hipGetLastError();
}

}  // namespace

int64_t gather_grid(int64_t rows, int topk, int64_t nbuckets, int item_pairs) {
  const int64_t max_items = (rows * topk + item_pairs - 1) / item_pairs + nbuckets;
  return (max_items + kXcds - 1) / kXcds * kXcds;
}

int gather_segments(int n, int d, int topk, bsa_dtype dtype) {
  if (n % 256 != 0) return 1;
  const int nb = n / kTile;
  const int64_t qbytes = static_cast<int64_t>(n) * d * (dtype == BSA_BF16 ? 2 : 4);
  int qs = 1;
  // halve the segment while its Q is over 4 MB (one XCD's L2), its length
  // stays a multiple of 256 rows, and a (segment, block) bucket still
  // averages >= 256 pairs.  Smaller segments trade query-row misses for
  // re-reads of the key blocks; at N = 32k, d = 64 the attention kernel took
  // 0.160 ms with one 4 MB segment per head, 0.163 with 2 MB and 0.169 with
  // 1 MB.  (Before the partial rows carried their own log-sum-exp, the
  // scattered 8-byte (m, l) stores evicted query rows from L2 and 2 MB
  // segments were best.)
  while (n % (qs * 2 * 256) == 0 && qbytes / qs > (int64_t(4) << 20) &&
         static_cast<int64_t>(n / (qs * 2)) * topk / nb >= 256)
    qs *= 2;
  return qs;
}

size_t gather_pair_bytes(int d, bsa_dtype dtype) {
  return static_cast<size_t>(d) * (dtype == BSA_BF16 ? 2 : 4);
}

hipError_t launch_gather_index(const GatherArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  const ChunkGeom c(a, row0, rows);
  if (a.ws.count_words > 0)  // counts not known to be zero (new buffer, or a failed launch)
    hipLaunchKernelGGL(zero_i32_kernel, dim3(static_cast<unsigned>((a.ws.count_words + 255) / 256)), dim3(256),
                       0, s, a.ws.count, a.ws.count_words);
  const int seg = a.n / a.qsegs;
  // Rows per bucketing workgroup: 256 (fewer global atomics) when that still
  // gives >= 512 workgroups and its LDS (histogram, bases and the ordered
  // records) lets two of them share a CU, else 128 under the same
  // conditions, else 64, so the whole GPU takes part.  (N = 4096, 8 heads:
  // bucketing 32 -> 24.5 us at 64 rows; N = 128k causal, 2048 blocks, k = 32:
  // 0.70 -> 0.56 ms per step at 128 rows, where 256 rows took 82 KB, one
  // workgroup per CU.)
  auto lds_for = [&](int r) {
    const int np_r = r * a.topk;
    return (2 * static_cast<size_t>(c.nb) + 4) * 4 + (np_r <= 256 * kPairRegs ? static_cast<size_t>(np_r) * 8 : 0);
  };
  int rpw = kTile;
  for (const int r : {256, 128})
    if (seg % r == 0 && row0 % r == 0 && rows >= int64_t(512) * r && lds_for(r) <= 80 * 1024) {
      rpw = r;
      break;
    }
  const int64_t row_groups = (rows + rpw - 1) / rpw;
  const size_t count_lds = lds_for(rpw);
  if (count_lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(bucket_count_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(count_lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bucket_count_kernel, dim3(static_cast<unsigned>(row_groups)), dim3(256),
                     count_lds, s, a.idx, a.ws.count, a.ws.rank, a.ws.rec,
                     a.ws.wg_valid, row0, rows, a.n, a.topk, a.causal, c.bh0, rpw, a.qsegs, a.seqtab);
  if (c.nbuckets <= kScanSmallMax)
    hipLaunchKernelGGL(bucket_scan_small_kernel, dim3(1), dim3(1024), 0, s, a.ws.count, a.ws.offsets, a.ws.items,
                       c.nbuckets, a.item_pairs);
  else
    hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(1024), 0, s, a.ws.count, a.ws.offsets,
                       a.ws.items, c.nbuckets, a.item_pairs);
  const int64_t bucket_groups = (c.nbuckets + 255) / 256;
  // the list starts of a (head, segment) go to LDS when they fit in 16 KB
  const int stage_off = c.nb <= 4096 ? 1 : 0;
  hipLaunchKernelGGL(bucket_fill_kernel,
                     dim3(static_cast<unsigned>(row_groups > bucket_groups ? row_groups : bucket_groups)),
                     dim3(256), stage_off ? static_cast<size_t>(c.nb) * 4 : 0, s, a.idx, a.ws.rank, a.ws.rec,
                     a.ws.wg_valid, a.ws.offsets, a.ws.items, a.ws.item_rec, c.nbuckets,
                     gather_grid(rows, a.topk, c.nbuckets, a.item_pairs), a.ws.list, row0, rows, a.n, a.topk, c.bh0,
                     a.qsegs, a.item_pairs, rpw, a.seqtab, stage_off);
  return hipGetLastError();
}

hipError_t launch_gather_partial(const GatherArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  if (a.dtype == BSA_BF16)
    return a.d == 64 ? partial_chunk<bf16_bits, 64>(a, row0, rows, s)
                     : partial_chunk<bf16_bits, 128>(a, row0, rows, s);
  return a.d == 64 ? partial_chunk<float, 64>(a, row0, rows, s)
                   : partial_chunk<float, 128>(a, row0, rows, s);
}

hipError_t launch_gather_combine(const GatherArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  if (a.dtype == BSA_BF16)
    return a.d == 64 ? combine_chunk<bf16_bits, 64>(a, row0, rows, s)
                     : combine_chunk<bf16_bits, 128>(a, row0, rows, s);
  return a.d == 64 ? combine_chunk<float, 64>(a, row0, rows, s)
                   : combine_chunk<float, 128>(a, row0, rows, s);
}

}  // namespace bsa
