// sparse_flash_fwd.hip -- Stage 2, fused fine attention over a per-query-tile
// list of 64-key tiles with per-row masks.
//
// What it computes (nishantmodi.me "sparse-attention-triton-bench", sections
// "Stage 2: fine attention" and "The Triton kernel"): for each query i,
// o_i = sum_j softmax_j(scale * q_i . k_j) v_j over the keys j visible to i,
// with an online softmax: running max m, running sum l and an unnormalised
// accumulator, rescaled as each key tile arrives, so no score ever leaves the
// chip.  Invisible keys take no part (score -inf; yayme/CUDA-kernel README,
// the note on masked keys).  A row with no visible key gets zeros.
//
// Tile sources:
//   dynamic -- the tile list of a 64-query tile is the union of its rows'
//     selected blocks (ascending), and row r sees block beta iff beta is in
//     its own selection; in the causal variant keys after the query are
//     hidden (only the diagonal block can hold such keys).
//   static  -- a CSR list of key tiles per query tile plus optional per-row
//     64-bit key masks, built on the host (the README's plan of precomputing
//     the active (row tile, column tile) list; infra.bea.ai "Block-Sparse &
//     Linear Attention Kernels", the loop over K/V blocks where the mask is set).
//     The list is cut on the host into work items of at most S key tiles of
//     one query tile, heaviest first (infra.bea.ai, section 4, the challenges
//     table: load imbalance answered by dynamic block scheduling).  A query
//     tile whose list fits one item is written directly; the items of a
//     longer list each write a split-softmax partial (the normalised rows and
//     their log-sum-exp), and static_combine merges them.
//
// Work layout (gfx950): a 256-thread workgroup owns 64 queries, 16 per wave.
// Each key tile (64 keys) is staged once into LDS for all four waves: K in its
// natural [key][d] layout, V transposed to [d][key] for bf16.  A wave whose 16
// rows see nothing in a tile skips its MFMA work for that tile.  With
// S^T = K * Q^T on v_mfma_f32_16x16x32_bf16 a lane ends up holding scores of
// ONE query (column lane%16) for 16 keys, so the row max / sum need only
// in-lane work plus two xor shuffles, and the bf16-rounded probabilities are
// already laid out as the B operand of O^T = V^T * P^T.  l is summed from the
// same rounded probabilities that feed the PV product.  fp32 inputs use
// v_mfma_f32_16x16x4_f32 the same way with float probabilities.  The next
// tile's global loads are issued into registers before the current tile's
// MFMA work (register double buffering).
#include "bsa_device.hpp"
#include "bsa_launch.hpp"
#include "kv_tile.hpp"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Per-lane online-softmax state: query row = lane % 16 of this wave; the lane
// accumulates O[row][16*dt + 4*(lane/16) + jj].
template <int D>
struct RowState {
  f32x4 acc[D / 16];
  float m;  // running max of log2-scaled scores (identical in the row's 4 lanes)
  float l;  // this lane's share of the running sum
};

// One key tile for one wave.  `vis` gives the visibility of the lane's 16
// keys (bit 4*t + jj for key 16*t + 4*(lane/16) + jj).
template <typename T, int D, bool SKIP>
__device__ __forceinline__ void tile_step(RowState<D>& st, const T* ks, const T* vs,
                                          const void* qreg, uint32_t vis, float scale_log2,
                                          int lane) {
  using L = KvLayout<T, D>;
  const int g = lane >> 4, c16 = lane & 15;
  // SKIP (the static tile lists): keys 16 t .. 16 t + 15 that no row of the
  // wave sees (a sparse static tile: often one visible key column) cost no
  // MFMA work: their scores are masked below whatever they hold, and their
  // probabilities are 0.  The query-tile union sees whole blocks or none,
  // and its caller already skips blocks no row of the wave selected.
  bool sub[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) sub[t] = !SKIP || ballot(((vis >> (4 * t)) & 0xFu) != 0u) != 0ull;
  f32x4 s[4];
  if constexpr (L::kBf16) {
    const bf16x8* qb = static_cast<const bf16x8*>(qreg);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (!sub[t]) continue;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (16 * t + c16) * L::KPITCH + 8 * g + 32 * kk);
        s[t] = mfma_16x16x32_bf16(a, qb[kk], s[t]);
      }
    }
  } else {
    const float* qf = static_cast<const float*>(qreg);
    constexpr int KS = D / 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (!sub[t]) continue;
      const float* kr = ks + (16 * t + c16) * L::KPITCH + KS * g;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) s[t] = mfma_16x16x4_f32(kr[kk], qf[kk], s[t]);
    }
  }
  // Scale into log2 units and mask.
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float z = ((vis >> (4 * t + jj)) & 1u) ? s[t][jj] * scale_log2 : -INFINITY;
      s[t][jj] = z;
      mx = fmaxf(mx, z);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;  // all hidden so far: keep zeros
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_use);
  st.m = m_new;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) st.acc[dt] *= alpha;
  float lsum = 0.f;
  if constexpr (L::kBf16) {
    __bf16 pb[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        pb[t][jj] = f32_to_bf16(__builtin_amdgcn_exp2f(s[t][jj] - m_use));
        lsum += static_cast<float>(pb[t][jj]);
      }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (!sub[2 * kk] && !sub[2 * kk + 1]) continue;  // keys 32 kk .. 32 kk + 31: all p = 0
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
        st.acc[dt] = mfma_16x16x32_bf16(a, bp, st.acc[dt]);
      }
    }
  } else {
    float p[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        p[t][jj] = __builtin_amdgcn_exp2f(s[t][jj] - m_use);
        lsum += p[t][jj];
      }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (!sub[t]) continue;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        // one MFMA step covers keys 16 t + 4 g' + jj of the four lane groups
        if (SKIP && ballot(((vis >> (4 * t + jj)) & 1u) != 0u) == 0ull) continue;
        const T* vr = vs + (16 * t + 4 * g + jj) * L::VPITCH + c16;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
          st.acc[dt] = mfma_16x16x4_f32(vr[16 * dt], p[t][jj], st.acc[dt]);
      }
    }
  }
  st.l = st.l * alpha + lsum;
}

// W waves per workgroup own a query tile of TQ = 16 W rows (W = 4: one
// 64-row block; W = 1, 2: part of one).
template <typename T, int D, bool CAUSAL, int W>
__global__ __launch_bounds__(64 * W) void sparse_flash_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    float* __restrict__ out, float* __restrict__ lse, const int32_t* __restrict__ idx, int topk,
    int n, const int4* __restrict__ seqtab, float scale_log2) {
  constexpr int NTH = 64 * W, TQ = 16 * W;
  using L = KvLayout<T, D, NTH>;
  extern __shared__ __align__(16) unsigned char smem[];
  T* ks = reinterpret_cast<T*>(smem);
  T* vs = reinterpret_cast<T*>(smem + L::K_BYTES);
  uint64_t* rm = reinterpret_cast<uint64_t*>(smem + L::BYTES);  // dynamic: per-block row bits

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int nqt = n / TQ;
  const int nb = n / kTile;
  const int64_t bh = blockIdx.x / nqt;
  int qt = static_cast<int>(blockIdx.x % nqt);
  if (CAUSAL) qt = nqt - 1 - qt;  // heaviest query tiles first
  const int64_t tile_row = bh * n + static_cast<int64_t>(qt) * TQ;
  const int qblk = qt * TQ / kTile;  // the 64-row block holding the tile
  const int qoff = qt * TQ % kTile;  // the tile's first row inside that block
  const T* kb = k + bh * static_cast<int64_t>(n) * D;
  const T* vb = v + bh * static_cast<int64_t>(n) * D;

  // ---- the tile list: the union of the rows' selected blocks (entries are
  // relative to the first block lo of the tile's sequence)
  int32_t* list = reinterpret_cast<int32_t*>(rm + nb);
  int nlist;
  {
    int lo = 0, hi = nb;
    if (seqtab) {
      const int4 e = seqtab[qblk];
      lo = e.x;
      hi = e.y;
    }
    const int nbc = CAUSAL ? qblk + 1 : hi;  // blocks lo .. nbc - 1 can be visible to this tile
    int* count = reinterpret_cast<int*>(list + nb);
    for (int c = lo + tid; c < nbc; c += NTH) rm[c] = 0ull;
    __syncthreads();
    const int32_t* ib = idx + tile_row * topk;
    for (int e = tid; e < TQ * topk; e += NTH) {
      const int b = ib[e];
      if (b >= 0 && b < nbc - lo) atomicOr(reinterpret_cast<unsigned long long*>(&rm[lo + b]), 1ull << (e / topk));
    }
    __syncthreads();
    if (wave == 0) {
      int cnt = 0;
      for (int c0 = lo; c0 < nbc; c0 += 64) {
        const int c = c0 + lane;
        const bool f = c < nbc && rm[c] != 0ull;
        const uint64_t m = ballot(f);
        if (f) list[cnt + static_cast<int>(lanes_below(m))] = c;
        cnt += __popcll(m);
      }
      if (lane == 0) *count = cnt;
    }
    __syncthreads();
    nlist = *count;
  }
  auto tile_at = [&](int it) -> int {
    const int kt = list[it];
    return (kt >= 0 && kt < nb) ? kt : -1;
  };

  // ---- this lane's query row in registers (B operand of S^T = K Q^T)
  const int64_t qrow = tile_row + wave * 16 + c16;
  const int qlocal = wave * 16 + c16;
  union {
    bf16x8 b[D / 32];
    float f[D / 4];
  } qreg;
  if constexpr (L::kBf16) {
    const T* qp = q + qrow * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qreg.b[kk] = as_bf16x8(ld16(qp + 32 * kk));
  } else {
    const T* qp = q + qrow * D + (D / 4) * g;
#pragma unroll
    for (int e = 0; e < D / 4; e += 4) {
      const uint4 u = ld16(qp + e);
      qreg.f[e] = __uint_as_float(u.x);
      qreg.f[e + 1] = __uint_as_float(u.y);
      qreg.f[e + 2] = __uint_as_float(u.z);
      qreg.f[e + 3] = __uint_as_float(u.w);
    }
  }

  RowState<D> st;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) st.acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;

  KvRegs<T, D, NTH> regs;
  int cur = nlist > 0 ? tile_at(0) : -1;
  if (cur >= 0) kv_load<T, D, NTH>(regs, kb, vb, cur, tid);
  for (int it = 0; it < nlist; ++it) {
    __syncthreads();
    if (cur >= 0) kv_store<T, D, NTH>(regs, ks, vs, tid);
    __syncthreads();
    const int nxt = it + 1 < nlist ? tile_at(it + 1) : -1;
    if (nxt >= 0) kv_load<T, D, NTH>(regs, kb, vb, nxt, tid);
    if (cur >= 0) {
      uint32_t vis;
      bool any;
      {
        const uint64_t bits = rm[cur];
        any = ((bits >> (16 * wave)) & 0xFFFFull) != 0ull;
        vis = ((bits >> qlocal) & 1ull) ? 0xFFFFu : 0u;
        if (CAUSAL && cur == qblk) {
          // diagonal block: key 16t + 4g + jj visible iff it is <= the query
          uint32_t cm = 0u;
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              if (16 * t + 4 * g + jj <= qoff + qlocal) cm |= 1u << (4 * t + jj);
          vis &= cm;
        }
        const int klim = block_keys(seqtab, cur);
        if (klim < kTile) {
          // a sequence's partial last block: keys klim .. 63 are padding
          uint32_t km = 0u;
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              if (16 * t + 4 * g + jj < klim) km |= 1u << (4 * t + jj);
          vis &= km;
        }
      }
      if (any) tile_step<T, D, false>(st, ks, vs, &qreg, vis, scale_log2, lane);
    }
    cur = nxt;
  }

  // ---- normalise and store
  float lt = st.l + __shfl_xor(st.l, 16);
  lt += __shfl_xor(lt, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (lse && g == 0)  // natural-log log-sum-exp; st.m is in log2 units
    lse[qrow] = lt > 0.f ? (st.m + __log2f(lt)) * (1.0f / kLog2e) : -INFINITY;
  float* op = out + qrow * D + 4 * g;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const f32x4 a = st.acc[dt] * inv;
    *reinterpret_cast<float4*>(op + 16 * dt) = make_float4(a[0], a[1], a[2], a[3]);
  }
}

// Per-query gathering (nishantmodi.me "sparse-attention-triton-bench", "The
// Triton kernel": one program per (batch, head, query) that loads each
// selected block's keys and values and runs the online softmax over them).
// One wave per query row, four rows per workgroup, no MFMA and no sharing of
// a key block between queries: every (query, block) pair reads its block's
// K and V again (through L2).  Lane (r, c) of the wave takes the 16-byte
// column chunk c (CH chunks per row) of rows r, r + RG, ... of a block (RG =
// 64 / CH row groups): its partial dot products are summed over the CH
// lanes of its row group, each lane then holds the scores (and
// probabilities) of its own rows, multiplies them into its chunk of those
// V rows, and the output's chunks are summed over the row groups once at
// the end.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void per_query_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    float* __restrict__ out, float* __restrict__ lse, const int32_t* __restrict__ idx, int64_t rows,
    int topk, int n, const int4* __restrict__ seqtab, float scale_log2) {
  constexpr int E = 16 / sizeof(T);  // elements per chunk
  constexpr int CH = D / E;          // chunks per row
  constexpr int RG = 64 / CH;        // row groups
  constexpr int RPL = 64 / RG;       // rows per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const int c = lane % CH, r = lane / CH;
  const int64_t bh = row / n;
  const int qi = static_cast<int>(row % n);
  const RowBlocks rb = row_blocks(seqtab, row, n, CAUSAL);
  auto to_f = [](const uint4& u, float (&x)[E]) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      x[0] = __uint_as_float(u.x);
      x[1] = __uint_as_float(u.y);
      x[2] = __uint_as_float(u.z);
      x[3] = __uint_as_float(u.w);
    }
  };
  float qv[E];
  to_f(ld16(q + row * D + c * E), qv);
  const T* kb = k + bh * static_cast<int64_t>(n) * D;
  const T* vb = v + bh * static_cast<int64_t>(n) * D;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;  // log2-domain running max; the row group's share of the sum
  const int32_t* sel = idx + row * topk;
  for (int t = 0; t < topk; ++t) {
    const int beta = sel_block(sel[t], rb);
    if (beta < 0) continue;  // wave-uniform
    const int klim = block_keys(seqtab, beta);
    const int kmax = CAUSAL && beta == rb.own ? qi % kTile : kTile - 1;  // last visible key
    float s[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int j = r + RG * i;
      float kx[E];
      to_f(ld16(kb + (static_cast<int64_t>(beta) * kTile + j) * D + c * E), kx);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) d = __builtin_fmaf(qv[e], kx[e], d);
      s[i] = d;
    }
#pragma unroll
    for (int off = 1; off < CH; off <<= 1)
#pragma unroll
      for (int i = 0; i < RPL; ++i) s[i] += __shfl_xor(s[i], off);
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int j = r + RG * i;
      s[i] = (j < klim && j <= kmax) ? s[i] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[i]);
    }
#pragma unroll
    for (int off = CH; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float m_new = fmaxf(m, mx);  // finite: every live block has a visible key
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int j = r + RG * i;
      const float p = __builtin_amdgcn_exp2f(s[i] - m);
      l += p;  // the same in the CH lanes of the row group
      float vx[E];
      to_f(ld16(vb + (static_cast<int64_t>(beta) * kTile + j) * D + c * E), vx);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(p, vx[e], acc[e]);
    }
  }
#pragma unroll
  for (int off = CH; off < 64; off <<= 1) {
    l += __shfl_xor(l, off);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (r == 0) {
    float* dst = out + row * D + c * E;
#pragma unroll
    for (int e = 0; e < E; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    if (lse && c == 0) lse[row] = l > 0.f ? (m + __log2f(l)) * (1.0f / kLog2e) : -INFINITY;
  }
}

// The query operand of S^T = K Q^T for one lane: its row, the d slots of
// MFMA k-group lane / 16.
template <typename T, int D>
union QReg {
  bf16x8 b[D / 32];
  float f[D / 4];
};

template <typename T, int D>
__device__ __forceinline__ void load_qreg(QReg<T, D>& qr, const T* __restrict__ q, int64_t qrow, int g) {
  if constexpr (sizeof(T) == 2) {
    const T* qp = q + qrow * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qr.b[kk] = as_bf16x8(ld16(qp + 32 * kk));
  } else {
    const T* qp = q + qrow * D + (D / 4) * g;
#pragma unroll
    for (int e = 0; e < D / 4; e += 4) {
      const uint4 u = ld16(qp + e);
      qr.f[e] = __uint_as_float(u.x);
      qr.f[e + 1] = __uint_as_float(u.y);
      qr.f[e + 2] = __uint_as_float(u.z);
      qr.f[e + 3] = __uint_as_float(u.w);
    }
  }
}

// Static tile list, one work item per workgroup: item = {query tile, first
// list entry, number of entries, partial slot (-1: the query tile's whole
// list, written to out directly)}.  Workgroup w runs item w / bh of head
// w % bh, so the heaviest items of every head start first.  Rows and keys at
// or past nv (a sequence whose length is not a multiple of 64) do not exist:
// their loads are clamped into the sequence, their keys masked, their rows
// not stored.  Partials: part[(bh * nslots + slot) * 64 + row] is the row's
// normalised output (D floats), part_lse the matching log2-domain
// log-sum-exp (-inf for a row that saw no key in the item).
template <typename T, int D>
__global__ __launch_bounds__(256) void static_item_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, float* __restrict__ out,
    const int4* __restrict__ items, int64_t bh_count, const int32_t* __restrict__ col,
    const uint64_t* __restrict__ rowmask, float* __restrict__ part, float* __restrict__ part_lse, int nslots,
    int nv, float scale_log2) {
  using L = KvLayout<T, D>;
  __shared__ __align__(16) unsigned char smem[L::BYTES];
  T* ks = reinterpret_cast<T*>(smem);
  T* vs = reinterpret_cast<T*>(smem + L::K_BYTES);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int nt = (nv + kTile - 1) / kTile;
  const int klast = nv - (nt - 1) * kTile;  // keys of the last tile
  const int4 it = items[blockIdx.x / bh_count];
  const int64_t bh = blockIdx.x % bh_count;
  const int qt = it.x, p0 = it.y, cnt = it.z, slot = it.w;
  const int64_t head = bh * static_cast<int64_t>(nv);
  const T* kb = k + head * D;
  const T* vb = v + head * D;
  const int qlocal = wave * 16 + c16;
  const int qi = qt * kTile + qlocal;  // row inside the sequence
  const bool row_ok = qi < nv;

  QReg<T, D> qreg;
  load_qreg<T, D>(qreg, q, head + (row_ok ? qi : nv - 1), g);
  RowState<D> st;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) st.acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;

  auto tile_at = [&](int e) -> int { return col[p0 + e]; };
  KvRegs<T, D> regs;
  int cur = cnt > 0 ? tile_at(0) : -1;
  if (cur >= 0) kv_load<T, D>(regs, kb, vb, cur, tid, cur == nt - 1 ? klast : kTile);
  for (int e = 0; e < cnt; ++e) {
    __syncthreads();
    kv_store<T, D>(regs, ks, vs, tid);
    __syncthreads();
    const int nxt = e + 1 < cnt ? tile_at(e + 1) : -1;
    if (nxt >= 0) kv_load<T, D>(regs, kb, vb, nxt, tid, nxt == nt - 1 ? klast : kTile);
    uint64_t m64 = rowmask ? rowmask[static_cast<int64_t>(p0 + e) * kTile + qlocal] : ~0ull;
    if (cur == nt - 1 && klast < kTile) m64 &= (1ull << klast) - 1ull;  // keys past the sequence
    if (!row_ok) m64 = 0ull;
    const bool any = ballot(m64 != 0ull) != 0ull;
    uint32_t vis = 0u;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        vis |= static_cast<uint32_t>((m64 >> (16 * t + 4 * g + jj)) & 1ull) << (4 * t + jj);
    if (any) tile_step<T, D, true>(st, ks, vs, &qreg, vis, scale_log2, lane);
    cur = nxt;
  }

  float lt = st.l + __shfl_xor(st.l, 16);
  lt += __shfl_xor(lt, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (!row_ok) return;
  float* op;
  if (slot < 0) {
    op = out + (head + qi) * D + 4 * g;
  } else {
    const int64_t prow = (bh * nslots + slot) * kTile + qlocal;
    op = part + prow * D + 4 * g;
    if (g == 0) part_lse[prow] = lt > 0.f ? st.m + __log2f(lt) : -INFINITY;
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const f32x4 a = st.acc[dt] * inv;
    *reinterpret_cast<float4*>(op + 16 * dt) = make_float4(a[0], a[1], a[2], a[3]);
  }
}

// Merge the partials of the query tiles whose list was split: split entry s
// = {query tile, first slot, number of slots}.  Four lanes per row, D/4 dims
// each; weights 2^(L_s - max L) in slot order.
template <int D>
__global__ __launch_bounds__(256) void static_combine_kernel(const int4* __restrict__ split, int64_t bh_count,
                                                             const float* __restrict__ part,
                                                             const float* __restrict__ part_lse, int nslots,
                                                             float* __restrict__ out, int nv) {
  constexpr int E = D / 4;
  const int4 sp = split[blockIdx.x / bh_count];
  const int64_t bh = blockIdx.x % bh_count;
  const int r = threadIdx.x >> 2, c = threadIdx.x & 3;
  const int qi = sp.x * kTile + r;
  if (qi >= nv) return;
  float mx = -INFINITY;
  for (int s = 0; s < sp.z; ++s) mx = fmaxf(mx, part_lse[(bh * nslots + sp.y + s) * kTile + r]);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (mx > -INFINITY) {
    for (int s = 0; s < sp.z; ++s) {
      const int64_t prow = (bh * nslots + sp.y + s) * kTile + r;
      const float ls = part_lse[prow];
      if (ls == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(ls - mx);
      wsum += w;
      const float* src = part + prow * D + c * E;
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const float4 x = *reinterpret_cast<const float4*>(src + e);
        acc[e] += w * x.x;
        acc[e + 1] += w * x.y;
        acc[e + 2] += w * x.z;
        acc[e + 3] += w * x.w;
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  float* dst = out + (bh * static_cast<int64_t>(nv) + qi) * D + c * E;
#pragma unroll
  for (int e = 0; e < E; e += 4)
    *reinterpret_cast<float4*>(dst + e) = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv,
                                                      acc[e + 3] * inv);
}

template <typename T, int D, bool CAUSAL, int W>
hipError_t launch_union(const void* q, const void* k, const void* v, float* out, float* lse,
                        const int32_t* idx, int topk, const int4* seqtab, int64_t bh, int n, float scale,
                        hipStream_t s) {
  using L = KvLayout<T, D, 64 * W>;
  const int nb = n / kTile;
  const size_t smem = L::BYTES + static_cast<size_t>(nb) * 8 + static_cast<size_t>(nb) * 4 + 16;
  const auto kern = sparse_flash_kernel<T, D, CAUSAL, W>;
  if (smem > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(smem));
    if (e != hipSuccess) return e;
  }
  const dim3 grid(static_cast<unsigned>(bh * (n / (16 * W))));
  hipLaunchKernelGGL(kern, grid, dim3(64 * W), smem, s, static_cast<const T*>(q),
                     static_cast<const T*>(k), static_cast<const T*>(v), out, lse, idx, topk, n, seqtab,
                     scale * kLog2e);
  return hipGetLastError();
}

template <typename T, int D, int W>
hipError_t dispatch_w(const void* q, const void* k, const void* v, float* out, float* lse,
                      const int32_t* idx, int64_t bh, int n, int topk, float scale,
                      int causal, hipStream_t s, const int4* seqtab) {
  return causal ? launch_union<T, D, true, W>(q, k, v, out, lse, idx, topk, seqtab, bh, n, scale, s)
                : launch_union<T, D, false, W>(q, k, v, out, lse, idx, topk, seqtab, bh, n, scale, s);
}

template <typename T, int D>
hipError_t dispatch_dynamic(const void* q, const void* k, const void* v, float* out, float* lse,
                            const int32_t* idx, int64_t bh, int n, int topk, float scale,
                            int causal, hipStream_t s, const int4* seqtab, int rows) {
  if (rows == 16) return dispatch_w<T, D, 1>(q, k, v, out, lse, idx, bh, n, topk, scale, causal, s, seqtab);
  if (rows == 32) return dispatch_w<T, D, 2>(q, k, v, out, lse, idx, bh, n, topk, scale, causal, s, seqtab);
  return dispatch_w<T, D, 4>(q, k, v, out, lse, idx, bh, n, topk, scale, causal, s, seqtab);
}

template <typename T, int D>
hipError_t launch_static_t(const StaticLaunch& a, hipStream_t s) {
  if (a.nitems > 0)
    hipLaunchKernelGGL((static_item_kernel<T, D>), dim3(static_cast<unsigned>(a.nitems * a.bh)), dim3(256), 0,
                       s, static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       a.out, a.items, a.bh, a.col, a.rowmask, a.part, a.part_lse, a.nslots, a.n,
                       a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_flash_dynamic(const void* q, const void* k, const void* v, float* out,
                                       float* lse, const int32_t* idx, int64_t bh, int n, int d,
                                       int topk, float scale, int causal, bsa_dtype dtype,
                                       hipStream_t stream, const int4* kl, int rows) {
  if (dtype == BSA_BF16)
    return d == 64 ? dispatch_dynamic<bf16_bits, 64>(q, k, v, out, lse, idx, bh, n, topk, scale, causal, stream, kl, rows)
                   : dispatch_dynamic<bf16_bits, 128>(q, k, v, out, lse, idx, bh, n, topk, scale, causal, stream, kl, rows);
  return d == 64 ? dispatch_dynamic<float, 64>(q, k, v, out, lse, idx, bh, n, topk, scale, causal, stream, kl, rows)
                 : dispatch_dynamic<float, 128>(q, k, v, out, lse, idx, bh, n, topk, scale, causal, stream, kl, rows);
}

hipError_t launch_sparse_flash_per_query(const void* q, const void* k, const void* v, float* out,
                                         float* lse, const int32_t* idx, int64_t rows, int n, int d,
                                         int topk, float scale, int causal, bsa_dtype dtype,
                                         hipStream_t stream, const int4* seqtab) {
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  const float sl2 = scale * kLog2e;
#define BSA_PQ(T, DD, C)                                                                                     \
  hipLaunchKernelGGL((per_query_kernel<T, DD, C>), grid, dim3(256), 0, stream, static_cast<const T*>(q),     \
                     static_cast<const T*>(k), static_cast<const T*>(v), out, lse, idx, rows, topk, n, seqtab, \
                     sl2)
  if (dtype == BSA_BF16) {
    if (d == 64) { if (causal) BSA_PQ(bf16_bits, 64, true); else BSA_PQ(bf16_bits, 64, false); }
    else { if (causal) BSA_PQ(bf16_bits, 128, true); else BSA_PQ(bf16_bits, 128, false); }
  } else {
    if (d == 64) { if (causal) BSA_PQ(float, 64, true); else BSA_PQ(float, 64, false); }
    else { if (causal) BSA_PQ(float, 128, true); else BSA_PQ(float, 128, false); }
  }
#undef BSA_PQ
  return hipGetLastError();
}

hipError_t launch_sparse_flash_static(const StaticLaunch& a, hipStream_t stream) {
  if (a.dtype == BSA_BF16)
    return a.d == 64 ? launch_static_t<bf16_bits, 64>(a, stream) : launch_static_t<bf16_bits, 128>(a, stream);
  return a.d == 64 ? launch_static_t<float, 64>(a, stream) : launch_static_t<float, 128>(a, stream);
}

hipError_t launch_static_combine(const StaticLaunch& a, hipStream_t stream) {
  if (a.nsplit <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(a.nsplit * a.bh));
  if (a.d == 64)
    hipLaunchKernelGGL((static_combine_kernel<64>), grid, dim3(256), 0, stream, a.split, a.bh, a.part, a.part_lse,
                       a.nslots, a.out, a.n);
  else
    hipLaunchKernelGGL((static_combine_kernel<128>), grid, dim3(256), 0, stream, a.split, a.bh, a.part,
                       a.part_lse, a.nslots, a.out, a.n);
  return hipGetLastError();
}

}  // namespace bsa
