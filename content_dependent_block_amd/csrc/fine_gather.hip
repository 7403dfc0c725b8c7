// fine_gather.hip -- Stage 2 by block-major gathering ("block-gather"):
// every selected (query, block) pair is computed exactly once on MFMA, with
// 16 pairs that share a key block packed into one MFMA tile.
//
// What it computes is the fine stage of nishantmodi.me
// "sparse-attention-triton-bench" (sections "Stage 2: fine attention" and
// "The Triton kernel"): o_i = softmax over the keys of query i's selected
// blocks, applied to V.  Instead of one online-softmax pass per query, the
// softmax is split by block (a standard split-softmax identity): each pair
// (i, beta) yields m = max of its log2-scaled scores, l = sum 2^(z - m), and
// o = (sum 2^(z - m) v) / l; the pairs of a query are then merged as
//   M = max m_s,  w_s = l_s 2^(m_s - M),  o_i = sum w_s o_s / sum w_s.
// No score leaves the chip; only the per-pair (m, l, o) do.
//
// Why: with content-dependent selections, queries that sit next to each other
// share few blocks, so a query tile's union of blocks is mostly work for one
// or two of its rows.  Grouping pairs by block instead gives full 16-row MFMA
// tiles and reads each K/V block once per 128 pairs.
//
// Kernels, per chunk of query rows (the chunk bounds the partial buffer):
//   bucket_count   -- histogram of the chunk's pairs by (head, block); each pair
//                     gets its rank inside its bucket (LDS histogram per 64 rows,
//                     one global atomic per (workgroup, block)).
//   bucket_scan    -- one workgroup: exclusive prefix of the counts (pair offsets)
//                     and of ceil(count / 128) (work-item offsets).
//   bucket_fill    -- pair ids into per-bucket lists.
//   gather_partial -- one work item = up to 128 pairs of one bucket: K and V^T
//                     of the block in LDS, the pairs' query rows gathered into
//                     MFMA operands, S^T = K Q^T and O^T = V^T P^T on MFMA,
//                     partial (m, l, o) out.  Work items are laid out so that
//                     consecutive items of one head land on one XCD.
//   combine        -- per query row, merge its partials in slot order.
// The order of pairs inside a bucket (set by atomics) does not affect any
// result: every MFMA column is computed independently of the others.
#include <type_traits>

#include "bsa_device.hpp"
#include "bsa_launch.hpp"

namespace bsa {
namespace {

constexpr int kItemPairs = 128;  // pairs per work item (8 groups of 16)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;

typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// A selection entry counts iff it names a real block and, in the causal
// variant, a block that is not after the query's own block.
__device__ __forceinline__ bool pair_valid(int beta, int nb, int64_t row, int n, int causal) {
  if (beta < 0 || beta >= nb) return false;
  return !causal || beta <= static_cast<int>(row % n) / kTile;
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int64_t count) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < count) p[i] = 0;
}

// One workgroup per 64 query rows (never straddles a head because n % 64 == 0).
__global__ __launch_bounds__(256) void bucket_count_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ count, int32_t* __restrict__ rank,
    int64_t row0, int64_t rows, int n, int topk, int causal, int64_t bh0) {
  extern __shared__ int32_t hist[];  // [nb] local counts, then [nb] global bases
  const int nb = n / kTile;
  int32_t* base = hist + nb;
  const int64_t r_begin = row0 + static_cast<int64_t>(blockIdx.x) * kTile;
  const int64_t nrows = (row0 + rows - r_begin) < kTile ? (row0 + rows - r_begin) : kTile;
  const int npairs = static_cast<int>(nrows) * topk;
  const int64_t p_begin = (r_begin - row0) * topk;  // chunk-relative pair id of the first pair
  const int64_t bucket0 = (r_begin / n - bh0) * nb;
  for (int c = threadIdx.x; c < nb; c += 256) hist[c] = 0;
  __syncthreads();
  for (int e = threadIdx.x; e < npairs; e += 256) {
    const int64_t row = r_begin + e / topk;
    const int beta = idx[row * topk + (e % topk)];
    rank[p_begin + e] = pair_valid(beta, nb, row, n, causal) ? atomicAdd(&hist[beta], 1) : -1;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < nb; c += 256)
    base[c] = hist[c] ? atomicAdd(&count[bucket0 + c], hist[c]) : 0;
  __syncthreads();
  for (int e = threadIdx.x; e < npairs; e += 256) {
    const int64_t row = r_begin + e / topk;
    const int32_t rk = rank[p_begin + e];
    if (rk >= 0) rank[p_begin + e] = base[idx[row * topk + (e % topk)]] + rk;
  }
}

// Single workgroup of 1024 threads.  offsets[b] / items[b] are exclusive
// prefixes; entry nbuckets holds the totals.
__global__ __launch_bounds__(1024) void bucket_scan_kernel(const int32_t* __restrict__ count,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ items,
                                                           int nbuckets) {
  __shared__ int32_t s_pairs[1024], s_items[1024];
  const int t = threadIdx.x;
  const int per = (nbuckets + 1023) / 1024;
  const int b0 = t * per;
  int32_t sp = 0, si = 0;
  for (int b = b0; b < b0 + per && b < nbuckets; ++b) {
    sp += count[b];
    si += (count[b] + kItemPairs - 1) / kItemPairs;
  }
  s_pairs[t] = sp;
  s_items[t] = si;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scan
    const int32_t ap = t >= off ? s_pairs[t - off] : 0;
    const int32_t ai = t >= off ? s_items[t - off] : 0;
    __syncthreads();
    s_pairs[t] += ap;
    s_items[t] += ai;
    __syncthreads();
  }
  int32_t rp = s_pairs[t] - sp, ri = s_items[t] - si;  // exclusive
  for (int b = b0; b < b0 + per && b < nbuckets; ++b) {
    offsets[b] = rp;
    items[b] = ri;
    rp += count[b];
    ri += (count[b] + kItemPairs - 1) / kItemPairs;
  }
  if (t == 1023) {
    offsets[nbuckets] = s_pairs[1023];
    items[nbuckets] = s_items[1023];
  }
}

__global__ __launch_bounds__(256) void bucket_fill_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ list, int64_t row0, int64_t npairs,
    int n, int topk, int64_t bh0) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (p >= npairs) return;
  const int32_t rk = rank[p];
  if (rk < 0) return;
  const int nb = n / kTile;
  const int64_t row = row0 + p / topk;
  const int beta = idx[row * topk + (p % topk)];
  const int64_t b = (row / n - bh0) * nb + beta;
  const int64_t pos = static_cast<int64_t>(offsets[b]) + rk;
  if (pos < npairs) list[pos] = static_cast<int32_t>(p);
}

template <typename T, int D>
struct GatherLayout {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int KPITCH = D + (kBf16 ? 8 : 4);
  static constexpr int VROWS = kBf16 ? D : kTile;
  static constexpr int VPITCH = kBf16 ? kTile + 4 : D + 4;
  static constexpr int K_BYTES = kTile * KPITCH * sizeof(T);
  static constexpr int V_BYTES = VROWS * VPITCH * sizeof(T);
  static constexpr int BYTES = K_BYTES + V_BYTES;
};

// Stage key block `beta` of head base pointers kb / vb into LDS (K as is,
// V transposed for bf16).
template <typename T, int D>
__device__ __forceinline__ void stage_block(const T* __restrict__ kb, const T* __restrict__ vb,
                                            int beta, T* ks, T* vs, int tid) {
  using L = GatherLayout<T, D>;
  const int64_t key0 = static_cast<int64_t>(beta) * kTile;
  if constexpr (L::kBf16) {
    for (int c = tid; c < kTile * D / 8; c += 256) {
      const int c8 = c % (D / 8), row = c / (D / 8);
      *reinterpret_cast<uint4*>(ks + row * L::KPITCH + c8 * 8) = ld16(kb + (key0 + row) * D + c8 * 8);
    }
    for (int it = tid; it < (kTile / 2) * (D / 8); it += 256) {
      const int c8 = it % (D / 8), p = it / (D / 8);
      const uint4 ra = ld16(vb + (key0 + 2 * p) * D + c8 * 8);
      const uint4 rb = ld16(vb + (key0 + 2 * p + 1) * D + c8 * 8);
      const uint32_t a[4] = {ra.x, ra.y, ra.z, ra.w};
      const uint32_t b[4] = {rb.x, rb.y, rb.z, rb.w};
      uint32_t* dst = reinterpret_cast<uint32_t*>(vs + (c8 * 8) * L::VPITCH + 2 * p);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[(2 * e) * (L::VPITCH / 2)] = (a[e] & 0xFFFFu) | (b[e] << 16);
        dst[(2 * e + 1) * (L::VPITCH / 2)] = (a[e] >> 16) | (b[e] & 0xFFFF0000u);
      }
    }
  } else {
    for (int c = tid; c < kTile * D / 4; c += 256) {
      const int c4 = c % (D / 4), row = c / (D / 4);
      *reinterpret_cast<uint4*>(ks + row * L::KPITCH + c4 * 4) = ld16(kb + (key0 + row) * D + c4 * 4);
      *reinterpret_cast<uint4*>(vs + row * L::VPITCH + c4 * 4) = ld16(vb + (key0 + row) * D + c4 * 4);
    }
  }
}

// bf16 inputs keep partial outputs as fp16 (|o| <= max |v|, relative error
// 2^-11), fp32 inputs as fp32.
template <typename T>
using PartialT = typename std::conditional<sizeof(T) == 2, f16, float>::type;

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void gather_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ list, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ items, int nbuckets, int64_t row0, int64_t npairs, int n,
    int topk, int64_t bh0, float scale_log2, PartialT<T>* __restrict__ po,
    float2* __restrict__ pml) {
  using L = GatherLayout<T, D>;
  __shared__ __align__(16) unsigned char smem[L::BYTES];
  __shared__ int s_bucket;
  T* ks = reinterpret_cast<T*>(smem);
  T* vs = reinterpret_cast<T*>(smem + L::K_BYTES);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;

  // Work item of this workgroup: consecutive items go to one XCD.
  const int total = items[nbuckets];
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int slot = static_cast<int>(blockIdx.x) / kXcds;
  if (slot >= per_xcd) return;
  const int item = (static_cast<int>(blockIdx.x) % kXcds) * per_xcd + slot;
  if (item >= total) return;
  if (tid == 0) {
    int lo = 0, hi = nbuckets - 1;  // last bucket with items[b] <= item
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (items[mid] <= item) lo = mid;
      else hi = mid - 1;
    }
    s_bucket = lo;
  }
  __syncthreads();
  const int b = s_bucket;
  const int nb = n / kTile;
  const int beta = b % nb;
  const int64_t bh = bh0 + b / nb;
  const int64_t first = static_cast<int64_t>(offsets[b]) + static_cast<int64_t>(item - items[b]) * kItemPairs;
  int64_t last = offsets[b + 1];
  if (last > npairs) last = npairs;
  const int cnt = first < last ? static_cast<int>((last - first) < kItemPairs ? (last - first) : kItemPairs) : 0;
  const T* kb = k + bh * static_cast<int64_t>(n) * D;
  const T* vb = v + bh * static_cast<int64_t>(n) * D;
  stage_block<T, D>(kb, vb, beta, ks, vs, tid);
  __syncthreads();

  for (int grp = wave; grp * 16 < cnt; grp += 4) {
    const int t = grp * 16 + c16;
    const bool live = t < cnt;
    int32_t pair = 0;
    if (live) pair = list[first + t];
    if (pair < 0 || pair >= npairs) pair = 0;
    const int64_t row = row0 + pair / topk;
    const int qi = static_cast<int>(row % n);
    // S^T = K Q^T: lane holds scores of its pair's query for keys 16t+4g+jj.
    f32x4 s[4];
    if constexpr (L::kBf16) {
      bf16x8 qb[D / 32];
      const T* qp = q + row * D + 8 * g;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) qb[kk] = live ? as_bf16x8(ld16(qp + 32 * kk)) : bf16x8{};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (16 * tt + c16) * L::KPITCH + 8 * g + 32 * kk);
          s[tt] = mfma_16x16x32_bf16(a, qb[kk], s[tt]);
        }
      }
    } else {
      constexpr int KS = D / 4;
      float qf[KS];
      const T* qp = q + row * D + KS * g;
#pragma unroll
      for (int e = 0; e < KS; e += 4) {
        const uint4 u = live ? ld16(qp + e) : uint4{0u, 0u, 0u, 0u};
        qf[e] = __uint_as_float(u.x);
        qf[e + 1] = __uint_as_float(u.y);
        qf[e + 2] = __uint_as_float(u.z);
        qf[e + 3] = __uint_as_float(u.w);
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const T* kr = ks + (16 * tt + c16) * L::KPITCH + KS * g;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) s[tt] = mfma_16x16x4_f32(kr[kk], qf[kk], s[tt]);
      }
    }
    const bool diag = CAUSAL && beta == qi / kTile;
    const int qlocal = qi % kTile;
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const bool vis = !diag || (16 * tt + 4 * g + jj) <= qlocal;
        const float z = vis ? s[tt][jj] * scale_log2 : -INFINITY;
        s[tt][jj] = z;
        mx = fmaxf(mx, z);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));  // >= 1 visible key per pair: finite
    f32x4 acc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    if constexpr (L::kBf16) {
      __bf16 pb[4][4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          pb[tt][jj] = f32_to_bf16(__builtin_amdgcn_exp2f(s[tt][jj] - mx));
          lsum += static_cast<float>(pb[tt][jj]);
        }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 bp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bp[i] = pb[2 * kk][i];
          bp[4 + i] = pb[2 * kk + 1][i];
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const T* vr = vs + (16 * dt + c16) * L::VPITCH + 32 * kk + 4 * g;
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + 16);
          const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[dt] = mfma_16x16x32_bf16(a, bp, acc[dt]);
        }
      }
    } else {
      float p[4][4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          p[tt][jj] = __builtin_amdgcn_exp2f(s[tt][jj] - mx);
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
    }
    float lt = lsum + __shfl_xor(lsum, 16);
    lt += __shfl_xor(lt, 32);
    if (live) {
      const float inv = 1.0f / lt;
      PartialT<T>* op = po + static_cast<int64_t>(pair) * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const f32x4 a = acc[dt] * inv;
        if constexpr (L::kBf16) {
          const f16x4 h = {static_cast<f16>(a[0]), static_cast<f16>(a[1]), static_cast<f16>(a[2]),
                           static_cast<f16>(a[3])};
          *reinterpret_cast<f16x4*>(op + 16 * dt) = h;
        } else {
          *reinterpret_cast<float4*>(op + 16 * dt) = make_float4(a[0], a[1], a[2], a[3]);
        }
      }
      if (g == 0) pml[pair] = make_float2(mx, lt);
    }
  }
}

// One group of 16 lanes per query row; lane holds D/16 consecutive dims.
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ idx,
                                                      const PartialT<T>* __restrict__ po,
                                                      const float2* __restrict__ pml,
                                                      float* __restrict__ out, int64_t row0,
                                                      int64_t rows, int n, int topk, int causal) {
  constexpr int E = D / 16;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  if (r >= rows) return;
  const int c = threadIdx.x & 15;
  const int64_t row = row0 + r;
  const int nb = n / kTile;
  const int32_t* sel = idx + row * topk;
  float mmax = -INFINITY;
  for (int s = 0; s < topk; ++s)
    if (pair_valid(sel[s], nb, row, n, causal)) mmax = fmaxf(mmax, pml[r * topk + s].x);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  for (int s = 0; s < topk; ++s) {
    if (!pair_valid(sel[s], nb, row, n, causal)) continue;
    const int64_t p = r * topk + s;
    const float2 ml = pml[p];
    const float w = ml.y * __builtin_amdgcn_exp2f(ml.x - mmax);
    wsum += w;
    const PartialT<T>* src = po + p * D + c * E;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const f16x4 h = *reinterpret_cast<const f16x4*>(src + e);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[e + u] += w * static_cast<float>(h[u]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const float4 f = *reinterpret_cast<const float4*>(src + e);
        acc[e] += w * f.x;
        acc[e + 1] += w * f.y;
        acc[e + 2] += w * f.z;
        acc[e + 3] += w * f.w;
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
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
    nbuckets = static_cast<int>((bh1 - bh0 + 1) * nb);
    npairs = rows * a.topk;
  }
};

template <typename T, int D>
hipError_t partial_chunk(const GatherArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  const ChunkGeom c(a, row0, rows);
  const int64_t max_items = (c.npairs + kItemPairs - 1) / kItemPairs + c.nbuckets;
  const int64_t grid = (max_items + kXcds - 1) / kXcds * kXcds;
  const float sl2 = a.scale * kLog2e;
  auto* po = reinterpret_cast<PartialT<T>*>(a.ws.partial_o);
  if (a.causal)
    hipLaunchKernelGGL((gather_partial_kernel<T, D, true>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, s, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.ws.list, a.ws.offsets, a.ws.items, c.nbuckets,
                       row0, c.npairs, a.n, a.topk, c.bh0, sl2, po, a.ws.partial_ml);
  else
    hipLaunchKernelGGL((gather_partial_kernel<T, D, false>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, s, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.ws.list, a.ws.offsets, a.ws.items, c.nbuckets,
                       row0, c.npairs, a.n, a.topk, c.bh0, sl2, po, a.ws.partial_ml);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t combine_chunk(const GatherArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  auto* po = reinterpret_cast<const PartialT<T>*>(a.ws.partial_o);
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0,
                     s, a.idx, po, a.ws.partial_ml, a.out, row0, rows, a.n, a.topk, a.causal);
  return hipGetLastError();
}

}  // namespace

size_t gather_pair_bytes(int d, bsa_dtype dtype) {
  return static_cast<size_t>(d) * (dtype == BSA_BF16 ? 2 : 4) + sizeof(float2);
}

hipError_t launch_gather_index(const GatherArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  const ChunkGeom c(a, row0, rows);
  hipLaunchKernelGGL(zero_i32_kernel, dim3(static_cast<unsigned>((c.nbuckets + 255) / 256)), dim3(256),
                     0, s, a.ws.count, static_cast<int64_t>(c.nbuckets));
  hipLaunchKernelGGL(bucket_count_kernel, dim3(static_cast<unsigned>((rows + kTile - 1) / kTile)),
                     dim3(256), static_cast<size_t>(c.nb) * 8, s, a.idx, a.ws.count, a.ws.rank, row0,
                     rows, a.n, a.topk, a.causal, c.bh0);
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(1024), 0, s, a.ws.count, a.ws.offsets,
                     a.ws.items, c.nbuckets);
  hipLaunchKernelGGL(bucket_fill_kernel, dim3(static_cast<unsigned>((c.npairs + 255) / 256)), dim3(256),
                     0, s, a.idx, a.ws.rank, a.ws.offsets, a.ws.list, row0, c.npairs, a.n, a.topk,
                     c.bh0);
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
