// fine_backward.hip -- backward of the fine stage with the selection held
// fixed (nishantmodi.me "sparse-attention-triton-bench", section "What's
// next": a backward pass through the softmax-weighted sum over the selected
// blocks, FlashAttention-2's recomputing backward as the dense model).
//
// With z_ij = scale * q_i.k_j over query i's visible keys J(i), the forward's
// per-row log-sum-exp lse_i, and the incoming gradient dO:
//   p_ij  = exp(z_ij - lse_i)                (recomputed, never stored)
//   dp_ij = dO_i . v_j,  delta_i = dO_i . o_i  (= sum_j p_ij dp_ij)
//   ds_ij = p_ij (dp_ij - delta_i)
//   dq_i  = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
//   dv_j  = sum_i p_ij dO_i.
//
// The work runs on the block-gather bucketing of the forward: one work item
// is up to bwd_item_pairs(d) (query, block) pairs that share key block beta, so
// K and V of the block are staged once and every pair reuses them.  Per tile
// of 64 pairs (16 per wave, one pair per MFMA column):
//   S^T = K Q^T and dP^T = V dO^T on MFMA (64 keys x 16 pairs per wave),
//   P^T, dS^T in registers,
//   dQ^T = K^T dS^T on MFMA: the pair's dq contribution from this block, one
//         row per pair (rounded to bf16 for bf16 inputs), summed per query
//         by bwd_dq in slot order (the same bits on every call);
//   dV += P^T dO and dK += dS^T Q on MFMA, each wave owning 16 keys of the
//         block and summing over all 64 pairs of the tile (P^T, dS^T, dO,
//         Q pass through LDS).
// At the end of the item its dk, dv (64 keys x d each) go to a per-item
// buffer; bwd_dkv sums the items of every (head, block) in item order.  No
// floating-point atomics anywhere; dk and dv still depend in their last bits
// on the order the bucketing's integer atomics give a block's pairs.
//
// bf16 inputs: MFMA operands in bf16 (P, dS and dO rounded to bf16 as the
// forward rounds P), fp32 accumulation and outputs.  fp32 inputs: fp32 MFMA
// throughout.
#include "bsa_device.hpp"
#include "bsa_launch.hpp"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;

// ---------------------------------------------------------------- prep --
// ld[row] = (lse * log2 e, sum_d dout * out): 16 lanes per row.
// For bf16 inputs it also writes dout rounded to bf16 (dout_b, [rows][D]),
// the operand the pair kernel gathers (half the bytes of the fp32 rows).
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const float* __restrict__ out,
                                                       const float* __restrict__ dout,
                                                       const float* __restrict__ lse,
                                                       float2* __restrict__ ld,
                                                       bf16_bits* __restrict__ dout_b, int64_t rows) {
  constexpr int E = D / 16;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  float s = 0.f;
  if (r < rows) {
    const float* o = out + r * D + c * E;
    const float* g = dout + r * D + c * E;
    uint32_t packed[E / 2];
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const float4 a = *reinterpret_cast<const float4*>(o + e);
      const float4 b = *reinterpret_cast<const float4*>(g + e);
      s += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
      packed[e / 2] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, f32_to_bf16(b.x))) |
                      (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, f32_to_bf16(b.y))) << 16);
      packed[e / 2 + 1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, f32_to_bf16(b.z))) |
                          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, f32_to_bf16(b.w))) << 16);
    }
    if (dout_b) {
      bf16_bits* dst = dout_b + r * D + c * E;
      if constexpr (E == 8)
        *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      else
        *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 16);
  if (r < rows && c == 0) ld[r] = make_float2(lse[r] * kLog2e, s);
}

// -------------------------------------------------------- LDS layout --
template <typename T, int D>
struct BwdLayout {
  static constexpr bool kBf16 = sizeof(T) == 2;
  // Workgroups per CU the kernel is sized for (waves per SIMD): bf16 d = 64
  // runs three (51 KB of LDS single-buffered, <= 168 VGPRs), bf16 d = 128
  // two (80 KB with 8-element row pads, <= 256 VGPRs); fp32 one or two.
  static constexpr int kWaves = !kBf16 ? 1 : D == 64 ? 3 : 2;
  static constexpr int PAD = kBf16 ? (D == 128 ? 8 : 16) : 4;
  // K, V natural [64 keys][KP]; bf16 also K^T [D][KTP key positions], the
  // keys of each row in the order ktpos gives.
  static constexpr int KP = D + PAD;
  static constexpr int KTP = kTile + (kBf16 ? PAD : 16);
  // P^T or dS^T [64 keys][PP pairs].
  static constexpr int PP = kTile + PAD;
  // bf16: dO^T or Q^T [D][PP pairs]; fp32: dO or Q natural [64 pairs][KP].
  static constexpr int K_BYTES = kTile * KP * sizeof(T);
  static constexpr int KT_BYTES = kBf16 ? D * KTP * 2 : 0;
  static constexpr int P_BYTES = kTile * PP * sizeof(T);
  static constexpr int O_BYTES = kBf16 ? D * PP * 2 : kTile * KP * 4;
  static constexpr int OFF_V = K_BYTES;
  static constexpr int OFF_KT = 2 * K_BYTES;
  static constexpr int OFF_P = OFF_KT + KT_BYTES;
  // Dual: separate buffers for the dV operands (P^T, dO) and the dK operands
  // (dS^T, Q), so a tile needs two barriers instead of four; used when both
  // fit in the CU's 160 KB of LDS at kWaves workgroups.
  static constexpr int SINGLE = OFF_P + P_BYTES + O_BYTES;
  static constexpr bool kDual = (SINGLE + P_BYTES + O_BYTES) * kWaves <= 160 * 1024;
  static constexpr int OFF_P2 = OFF_P + P_BYTES;                   // dual only
  static constexpr int OFF_O = OFF_P + (kDual ? 2 : 1) * P_BYTES;
  static constexpr int OFF_O2 = OFF_O + O_BYTES;                   // dual only
  static constexpr int BYTES = OFF_O + (kDual ? 2 : 1) * O_BYTES;
  static_assert(BYTES * kWaves <= 160 * 1024, "kWaves workgroups fit a CU's LDS");
};

// Position of key k inside a K^T row: within each group of 32 keys, key
// 16h + 4g + i (h < 2, g < 4, i < 4) sits at 8g + 4h + i, so the eight keys
// lane group g feeds to one k-step of dQ^T = K^T dS^T (4g .. 4g+3 and
// 16 + 4g .. 16 + 4g + 3, the order of S^T's C layout) are one aligned
// 16-byte read.  Keys 2p and 2p + 1 stay adjacent.
__device__ __forceinline__ int ktpos(int k) {
  return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

// K and V of one key block into LDS (K natural and, for bf16, transposed;
// V natural).  bf16: every thread moves keys (2p, 2p+1) x 8 dims, so K^T gets
// two keys per 32-bit LDS write.  fp32: 16-byte pieces of key rows.
template <typename T, int D>
__device__ __forceinline__ void stage_kv(const T* __restrict__ kb, const T* __restrict__ vb, T* ks,
                                         T* vs, T* kt, int tid) {
  using L = BwdLayout<T, D>;
  if constexpr (L::kBf16) {
#pragma unroll
    for (int u = 0; u < D / 64; ++u) {
      const int it = tid + 256 * u, c8 = it % (D / 8), p = it / (D / 8);
      const uint4 k0 = ld16(kb + (2 * p) * D + c8 * 8), k1 = ld16(kb + (2 * p + 1) * D + c8 * 8);
      const uint4 v0 = ld16(vb + (2 * p) * D + c8 * 8), v1 = ld16(vb + (2 * p + 1) * D + c8 * 8);
      *reinterpret_cast<uint4*>(ks + (2 * p) * L::KP + c8 * 8) = k0;
      *reinterpret_cast<uint4*>(ks + (2 * p + 1) * L::KP + c8 * 8) = k1;
      *reinterpret_cast<uint4*>(vs + (2 * p) * L::KP + c8 * 8) = v0;
      *reinterpret_cast<uint4*>(vs + (2 * p + 1) * L::KP + c8 * 8) = v1;
      const uint32_t a[4] = {k0.x, k0.y, k0.z, k0.w};
      const uint32_t b[4] = {k1.x, k1.y, k1.z, k1.w};
      uint32_t* dst = reinterpret_cast<uint32_t*>(kt + (c8 * 8) * L::KTP + ktpos(2 * p));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // dim c8*8 + 2e (low halves) and + 2e + 1 (high halves); keys 2p, 2p+1
        dst[(2 * e) * (L::KTP / 2)] = (a[e] & 0xFFFFu) | (b[e] << 16);
        dst[(2 * e + 1) * (L::KTP / 2)] = (a[e] >> 16) | (b[e] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      const int c = tid + 256 * u, c4 = c % (D / 4), row = c / (D / 4);
      *reinterpret_cast<uint4*>(ks + row * L::KP + c4 * 4) = ld16(kb + row * D + c4 * 4);
      *reinterpret_cast<uint4*>(vs + row * L::KP + c4 * 4) = ld16(vb + row * D + c4 * 4);
    }
  }
}

// The pair's query row and incoming-gradient row as MFMA B operands.
// bf16: slot group g = lane/16 holds dims 32kk + 8g .. +7 of k-step kk.
// fp32: group g holds dims (D/4) g .. (D/4) g + D/4 - 1, one per k-step.
template <typename T, int D>
struct PairRows {
  static constexpr bool kBf16 = sizeof(T) == 2;
  bf16x8 qb[kBf16 ? D / 32 : 1];
  bf16x8 ob[kBf16 ? D / 32 : 1];
  float qf[kBf16 ? 1 : D / 4];
  float of[kBf16 ? 1 : D / 4];
};

// Raw inputs of the lane's pair for one tile, loaded a tile ahead of use:
// its query row and incoming-gradient row (the lane's dims as above), the
// row statistics, the row and the pair id.
template <typename T, int D>
struct PairIn {
  static constexpr int NQ = sizeof(T) == 2 ? D / 32 : D / 16;  // 16-byte pieces of q and of dout
  uint4 q[NQ];
  uint4 o[NQ];  // bf16: the bf16 copy of dout, dims 32kk + 8g .. +7; fp32: dims (D/4) g + 4i ..
  float2 lr;
  int64_t row;
  int32_t pair;
  bool live;
};

template <typename T, int D>
__device__ __forceinline__ void fetch(PairIn<T, D>& x, const T* __restrict__ q,
                                      const void* __restrict__ dout, const float2* __restrict__ ld,
                                      int32_t entry, bool live, int64_t row0, int64_t npairs,
                                      uint64_t div_magic, int div_shift, int g) {
  if (entry < 0 || entry >= npairs) live = false;
  x.live = live;
  x.pair = live ? entry : 0;
  x.row = row0 + static_cast<int64_t>((static_cast<uint64_t>(x.pair) * div_magic) >> div_shift);
#pragma unroll
  for (int i = 0; i < PairIn<T, D>::NQ; ++i) x.q[i] = x.o[i] = uint4{0u, 0u, 0u, 0u};
  if (live) {
    if constexpr (sizeof(T) == 2) {
      const bf16_bits* ob = static_cast<const bf16_bits*>(dout);
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const int d0 = 32 * kk + 8 * g;
        x.q[kk] = ld16(q + x.row * D + d0);
        x.o[kk] = ld16(ob + x.row * D + d0);
      }
    } else {
      constexpr int KS = D / 4;
      const float* of = static_cast<const float*>(dout);
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        x.q[i] = ld16(q + x.row * D + KS * g + 4 * i);
        x.o[i] = ld16(of + x.row * D + KS * g + 4 * i);
      }
    }
  }
  x.lr = live ? ld[x.row] : make_float2(0.f, 0.f);
}

template <typename T, int D>
__device__ __forceinline__ void ready(PairRows<T, D>& pr, const PairIn<T, D>& x) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      pr.qb[kk] = as_bf16x8(x.q[kk]);
      pr.ob[kk] = as_bf16x8(x.o[kk]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      pr.qf[4 * i] = __uint_as_float(x.q[i].x);
      pr.qf[4 * i + 1] = __uint_as_float(x.q[i].y);
      pr.qf[4 * i + 2] = __uint_as_float(x.q[i].z);
      pr.qf[4 * i + 3] = __uint_as_float(x.q[i].w);
      pr.of[4 * i] = __uint_as_float(x.o[i].x);
      pr.of[4 * i + 1] = __uint_as_float(x.o[i].y);
      pr.of[4 * i + 2] = __uint_as_float(x.o[i].z);
      pr.of[4 * i + 3] = __uint_as_float(x.o[i].w);
    }
  }
}

// One wave's 64 keys x 16 pairs: S^T = K Q^T and dP^T = V dO^T.
template <typename T, int D>
__device__ __forceinline__ void scores(const T* ks, const T* vs, const PairRows<T, D>& pr, f32x4 (&s)[4],
                                       f32x4 (&dp)[4], int g, int c16) {
  using L = BwdLayout<T, D>;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dp[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (L::kBf16) {
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const int off = (16 * tt + c16) * L::KP + 8 * g + 32 * kk;
        s[tt] = mfma_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(ks + off), pr.qb[kk], s[tt]);
        dp[tt] = mfma_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(vs + off), pr.ob[kk], dp[tt]);
      }
    } else {
      constexpr int KS = D / 4;
      const T* kr = ks + (16 * tt + c16) * L::KP + KS * g;
      const T* vr = vs + (16 * tt + c16) * L::KP + KS * g;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        s[tt] = mfma_16x16x4_f32(kr[kk], pr.qf[kk], s[tt]);
        dp[tt] = mfma_16x16x4_f32(vr[kk], pr.of[kk], dp[tt]);
      }
    }
  }
}

// One work item.  Workgroup = 4 waves; tiles of 64 pairs, wave w takes pairs
// 16w .. 16w + 15 of the tile (lane%16 = its pair), and owns keys
// 16w .. 16w + 15 of the block for dK and dV.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, (BwdLayout<T, D>::kWaves)) void bwd_pair_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const void* __restrict__ dout, const float2* __restrict__ ld,
    const int32_t* __restrict__ list, const int32_t* __restrict__ items,
    const int4* __restrict__ item_rec, int nbuckets, int64_t row0, int64_t npairs, int n,
    uint64_t div_magic, int div_shift, int64_t bh0, int qsegs, const int4* __restrict__ seqtab, float scale,
    float scale_log2, float* __restrict__ dq_part,
    float* __restrict__ dkv_part) {
  using L = BwdLayout<T, D>;
  extern __shared__ __align__(16) unsigned char smem[];
  T* ks = reinterpret_cast<T*>(smem);
  T* vs = reinterpret_cast<T*>(smem + L::OFF_V);
  T* kt = reinterpret_cast<T*>(smem + L::OFF_KT);
  T* pt = reinterpret_cast<T*>(smem + L::OFF_P);
  T* ot = reinterpret_cast<T*>(smem + L::OFF_O);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;

  const int total = items[nbuckets];
  const int4 rec = item_rec[blockIdx.x];
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int slot = static_cast<int>(blockIdx.x) / kXcds;
  const int item = (static_cast<int>(blockIdx.x) % kXcds) * per_xcd + slot;
  if (slot >= per_xcd || item >= total) return;  // whole workgroup: no item here
  const int b = rec.x;
  if (b < 0 || b >= nbuckets) return;
  const int64_t first = rec.y;
  int cnt = rec.z;
  if (cnt > bwd_item_pairs(D)) cnt = bwd_item_pairs(D);
  if (first + cnt > npairs) cnt = first < npairs ? static_cast<int>(npairs - first) : 0;
  const int nb = n / kTile;
  const int beta = b % nb;
  const int64_t bh = bh0 + b / (nb * qsegs);
  const int klim = block_keys(seqtab, beta);  // keys of the block that exist (the rest pad)

  stage_kv<T, D>(k + (bh * n + static_cast<int64_t>(beta) * kTile) * D,
                 v + (bh * n + static_cast<int64_t>(beta) * kTile) * D, ks, vs, kt, tid);

  f32x4 dk[D / 16], dv[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();

  const int ntiles = (cnt + 63) / 64;  // workgroup-uniform
  // Inputs run one tile ahead of the compute (list entries two tiles ahead),
  // so the gathered rows of tile it + 1 load while tile it computes.
  const int tl = 16 * wave + c16;  // the lane's pair position inside a tile
  int32_t ent = tl + 64 < cnt ? list[first + tl + 64] : 0;
  PairIn<T, D> cur;
  fetch<T, D>(cur, q, dout, ld, tl < cnt ? list[first + tl] : 0, tl < cnt, row0, npairs, div_magic,
              div_shift, g);
  for (int it = 0; it < ntiles; ++it) {
    PairIn<T, D> nxt;
    const int tn = (it + 1) * 64 + tl;
    fetch<T, D>(nxt, q, dout, ld, ent, tn < cnt, row0, npairs, div_magic, div_shift, g);
    ent = tn + 64 < cnt ? list[first + tn + 64] : 0;
    const bool live = cur.live;
    const int32_t pair = cur.pair;
    const int64_t row = cur.row;
    const float2 lr = cur.lr;
    PairRows<T, D> pr;
    ready<T, D>(pr, cur);

    f32x4 s[4], dp[4];
    scores<T, D>(ks, vs, pr, s, dp, g, c16);

    // P^T and dS^T of the lane's pair: keys 16tt + 4g + jj.
    const int qlocal = static_cast<int>(row % n) - beta * kTile;  // < 64 only on the diagonal
    float pv[4][4], dsv[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int key = 16 * tt + 4 * g + jj;
        const bool vis = live && (!CAUSAL || key <= qlocal) && key < klim;
        const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][jj], scale_log2, -lr.x)) : 0.f;
        pv[tt][jj] = p;
        dsv[tt][jj] = p * (dp[tt][jj] - lr.y);
      }

    // dQ^T = K^T dS^T: this block's contribution to the pair's dq, in two
    // halves of the output dims (half the accumulators live at a time).
    constexpr int DH = D / 32;  // 16-dim output tiles per half
    if constexpr (L::kBf16) {
      bf16x8 bs[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bs[kk][i] = f32_to_bf16(dsv[2 * kk][i]);
          bs[kk][4 + i] = f32_to_bf16(dsv[2 * kk + 1][i]);
        }
      // The pair's dq row, rounded to bf16 (fp32's range: no scale needed);
      // acc[t][e] = dq of dim 16 (DH h + t) + 4g + e (C layout: row 4g + e).
      uint16_t* dst = reinterpret_cast<uint16_t*>(dq_part) + static_cast<int64_t>(pair) * D + 4 * g;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 acc[DH];
#pragma unroll
        for (int t = 0; t < DH; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int t = 0; t < DH; ++t) {
            const int dt = DH * h + t;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + (16 * dt + c16) * L::KTP + 32 * kk + 8 * g);
            acc[t] = mfma_16x16x32_bf16(a, bs[kk], acc[t]);
          }
        if (live) {
#pragma unroll
          for (int t = 0; t < DH; ++t) {
            const f32x4 a = acc[t] * scale;
            const uint32_t lo = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, f32_to_bf16(a[0]))) |
                                (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, f32_to_bf16(a[1]))) << 16);
            const uint32_t hi = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, f32_to_bf16(a[2]))) |
                                (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, f32_to_bf16(a[3]))) << 16);
            *reinterpret_cast<uint2*>(dst + 16 * (DH * h + t)) = make_uint2(lo, hi);
          }
        }
      }
    } else {
      float* dst = dq_part + static_cast<int64_t>(pair) * D + 4 * g;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 acc[DH];
#pragma unroll
        for (int t = 0; t < DH; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const T* kr = ks + (16 * tt + 4 * g + jj) * L::KP + c16;
#pragma unroll
            for (int t = 0; t < DH; ++t) acc[t] = mfma_16x16x4_f32(kr[16 * (DH * h + t)], dsv[tt][jj], acc[t]);
          }
        if (live) {
#pragma unroll
          for (int t = 0; t < DH; ++t) {
            const f32x4 a = acc[t] * scale;
            *reinterpret_cast<float4*>(dst + 16 * (DH * h + t)) = make_float4(a[0], a[1], a[2], a[3]);
          }
        }
      }
    }

    // dV += P^T dO and dK += dS^T Q over the tile's 64 pairs: the lane's
    // column of P^T (or dS^T) and of dO (or Q) into LDS, then each wave's 16
    // keys against all 64 pairs.
    const int col = 16 * wave + c16;  // the lane's pair column in the tile
    auto put = [&](T* pbuf, T* obuf, int phase) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float x = phase == 0 ? pv[tt][jj] : dsv[tt][jj];
          if constexpr (L::kBf16)
            reinterpret_cast<__bf16*>(pbuf)[(16 * tt + 4 * g + jj) * L::PP + col] = f32_to_bf16(x);
          else
            pbuf[(16 * tt + 4 * g + jj) * L::PP + col] = x;
        }
      if constexpr (L::kBf16) {
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            reinterpret_cast<__bf16*>(obuf)[(32 * kk + 8 * g + i) * L::PP + col] =
                phase == 0 ? pr.ob[kk][i] : pr.qb[kk][i];
      } else {
        constexpr int KS = D / 4;
        float* orow = reinterpret_cast<float*>(obuf) + col * L::KP + KS * g;
#pragma unroll
        for (int e = 0; e < KS; e += 4) {
          if (phase == 0)
            *reinterpret_cast<float4*>(orow + e) = make_float4(pr.of[e], pr.of[e + 1], pr.of[e + 2], pr.of[e + 3]);
          else
            *reinterpret_cast<float4*>(orow + e) = make_float4(pr.qf[e], pr.qf[e + 1], pr.qf[e + 2], pr.qf[e + 3]);
        }
      }
    };
    auto mul = [&](const T* pbuf, const T* obuf, f32x4(&acc)[D / 16]) {
      if constexpr (L::kBf16) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(pbuf + (16 * wave + c16) * L::PP + 32 * kk + 8 * g);
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            const bf16x8 bb = *reinterpret_cast<const bf16x8*>(obuf + (16 * dt + c16) * L::PP + 32 * kk + 8 * g);
            acc[dt] = mfma_16x16x32_bf16(a, bb, acc[dt]);
          }
        }
      } else {
        const float* orows = reinterpret_cast<const float*>(obuf);
#pragma unroll 4
        for (int st = 0; st < 16; ++st) {
          const float a = pbuf[(16 * wave + c16) * L::PP + 4 * st + g];
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt)
            acc[dt] = mfma_16x16x4_f32(a, orows[(4 * st + g) * L::KP + 16 * dt + c16], acc[dt]);
        }
      }
    };
    if constexpr (L::kDual) {
      T* pt2 = reinterpret_cast<T*>(smem + L::OFF_P2);
      T* ot2 = reinterpret_cast<T*>(smem + L::OFF_O2);
      put(pt, ot, 0);
      put(pt2, ot2, 1);
      __syncthreads();
      mul(pt, ot, dv);
      mul(pt2, ot2, dk);
      __syncthreads();
    } else {
      put(pt, ot, 0);
      __syncthreads();
      mul(pt, ot, dv);
      __syncthreads();
      put(pt, ot, 1);
      __syncthreads();
      mul(pt, ot, dk);
      __syncthreads();
    }
    cur = nxt;
  }

  // The item's dk (scaled) and dv: [item][0 = dk, 1 = dv][64 keys][D].
  float* dst = dkv_part + static_cast<int64_t>(item) * 2 * kTile * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = 16 * wave + 4 * g + e, c = 16 * dt + c16;
      dst[key * D + c] = dk[dt][e] * scale;
      dst[(kTile + key) * D + c] = dv[dt][e];
    }
}

// dq[row] = sum over the row's valid slots, in slot order, of its pairs'
// contributions.  16 lanes per row, S slots at a time (16; 8 for fp32 rows
// at d = 128, whose 8 words per lane and slot would otherwise cost the
// kernel occupancy): every lane issues the loads of its D/16 dims of all S
// before adding any (slot index clamped into the row, so every load is in
// bounds), lane c < S decides whether slot s0 + c counts, and a ballot shares
// the answers with the row's lanes; slots that are padding were never
// written, and their words are zeroed before the sum.
// HALF: the rows are bf16 (bf16 inputs), else fp32.
template <int D, bool HALF>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const int32_t* __restrict__ idx,
                                                     const void* __restrict__ dq_part,
                                                     float* __restrict__ dq, int64_t row0,
                                                     int64_t rows, int n, int topk, int causal,
                                                     const int4* __restrict__ seqtab) {
  constexpr int E = D / 16;                // dims per lane
  constexpr int LW = HALF ? E / 2 : E;     // 32-bit words per lane and slot
  constexpr int WPR = HALF ? D / 2 : D;    // 32-bit words per contribution row
  constexpr int S = LW >= 8 ? 8 : 16;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  const int gbase = (threadIdx.x & 63) & ~15;
  const bool row_ok = r < rows;  // lanes of a missing row still take part in the ballot
  const int64_t rc = row_ok ? r : rows - 1;
  const int64_t row = row0 + rc;
  const RowBlocks rb = row_blocks(seqtab, row, n, causal);
  const uint32_t* src = static_cast<const uint32_t*>(dq_part) + rc * topk * WPR + c * LW;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < topk; s0 += S) {
    uint32_t w[S][LW];
#pragma unroll
    for (int t = 0; t < S; ++t) {
      const int st = s0 + t < topk ? s0 + t : topk - 1;
      const uint32_t* p = src + static_cast<int64_t>(st) * WPR;
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
    const bool valid = row_ok && c < S && s0 + c < topk && sel_block(idx[row * topk + s0 + c], rb) >= 0;
    const uint32_t vmask = static_cast<uint32_t>(ballot(valid) >> gbase) & 0xFFFFu;
#pragma unroll
    for (int t = 0; t < S; ++t) {
      const bool on = (vmask >> t) & 1u;
#pragma unroll
      for (int k2 = 0; k2 < LW; ++k2) {
        const uint32_t x = on ? w[t][k2] : 0u;
        if constexpr (HALF) {
          acc[2 * k2] += __uint_as_float(x << 16);
          acc[2 * k2 + 1] += __uint_as_float(x & 0xFFFF0000u);
        } else {
          acc[k2] += __uint_as_float(x);
        }
      }
    }
  }
  if (!row_ok) return;
  float* dst = dq + row * D + c * E;
#pragma unroll
  for (int e = 0; e < E; e += 4)
    *reinterpret_cast<float4*>(dst + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
}

// dk, dv of one (head, key block): the sum of its work items over the
// head's query segments, in item order.  Added to the existing values when
// the head's rows began before this chunk (an earlier chunk wrote them).
template <int D>
__global__ __launch_bounds__(256) void bwd_dkv_kernel(const float* __restrict__ dkv_part,
                                                      const int32_t* __restrict__ items,
                                                      float* __restrict__ dk, float* __restrict__ dv,
                                                      int64_t row0, int n, int64_t bh0, int qsegs) {
  constexpr int V = 2 * kTile * D / 4 / 256;  // float4 per thread
  const int nb = n / kTile;
  const int64_t hb = blockIdx.x / nb;  // head relative to bh0
  const int beta = static_cast<int>(blockIdx.x % nb);
  const int64_t bh = bh0 + hb;
  float4 acc[V];
#pragma unroll
  for (int u = 0; u < V; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sg = 0; sg < qsegs; ++sg) {
    const int64_t b = (hb * qsegs + sg) * nb + beta;
    for (int i = items[b]; i < items[b + 1]; ++i) {
      const float4* src = reinterpret_cast<const float4*>(dkv_part + static_cast<int64_t>(i) * 2 * kTile * D);
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const float4 x = src[threadIdx.x + 256 * u];
        acc[u].x += x.x;
        acc[u].y += x.y;
        acc[u].z += x.z;
        acc[u].w += x.w;
      }
    }
  }
  const bool add = bh * n < row0;
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int e4 = threadIdx.x + 256 * u;          // float4 index in [2][64][D]
    const int which = e4 / (kTile * D / 4);
    const int rem = e4 % (kTile * D / 4);
    float4* dst = reinterpret_cast<float4*>((which == 0 ? dk : dv) + (bh * n + static_cast<int64_t>(beta) * kTile) * D) + rem;
    float4 x = acc[u];
    if (add) {
      const float4 y = *dst;
      x.x += y.x;
      x.y += y.y;
      x.z += y.z;
      x.w += y.w;
    }
    *dst = x;
  }
}

struct Geom {
  int nb, nbuckets;
  int64_t bh0, bh1, npairs;
  Geom(const BackwardArgs& a, int64_t row0, int64_t rows) {
    nb = a.n / kTile;
    bh0 = row0 / a.n;
    bh1 = (row0 + rows - 1) / a.n;
    nbuckets = static_cast<int>((bh1 - bh0 + 1) * a.qsegs * nb);
    npairs = rows * a.topk;
  }
};

template <typename T, int D, bool CAUSAL>
hipError_t pairs_launch(const BackwardArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  using L = BwdLayout<T, D>;
  const Geom c(a, row0, rows);
  const int64_t grid = gather_grid(rows, a.topk, c.nbuckets, bwd_item_pairs(D));
  int lg = 0;
  while ((1 << lg) < a.topk) ++lg;
  const int shift = 32 + lg;
  const uint64_t magic = ((uint64_t(1) << shift) + uint64_t(a.topk) - 1) / uint64_t(a.topk);
  const auto kern = bwd_pair_kernel<T, D, CAUSAL>;
  if (L::BYTES > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(256), L::BYTES, s,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                     sizeof(T) == 2 ? static_cast<const void*>(a.dout_b) : static_cast<const void*>(a.dout),
                     a.ld, a.ws.list, a.ws.items, a.ws.item_rec, c.nbuckets, row0, c.npairs,
                     a.n, magic, shift, c.bh0, a.qsegs, a.seqtab, a.scale, a.scale * kLog2e,
                     a.dq_part, a.dkv_part);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t pairs_dispatch(const BackwardArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  return a.causal ? pairs_launch<T, D, true>(a, row0, rows, s) : pairs_launch<T, D, false>(a, row0, rows, s);
}

}  // namespace

hipError_t launch_bwd_prep(const BackwardArgs& a, int64_t rows, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((rows + 15) / 16));
  bf16_bits* ob = a.dtype == BSA_BF16 ? a.dout_b : nullptr;
  if (a.d == 64)
    hipLaunchKernelGGL(bwd_prep_kernel<64>, grid, dim3(256), 0, s, a.out, a.dout, a.lse, a.ld, ob, rows);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<128>, grid, dim3(256), 0, s, a.out, a.dout, a.lse, a.ld, ob, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_pairs(const BackwardArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  if (a.dtype == BSA_BF16)
    return a.d == 64 ? pairs_dispatch<bf16_bits, 64>(a, row0, rows, s)
                     : pairs_dispatch<bf16_bits, 128>(a, row0, rows, s);
  return a.d == 64 ? pairs_dispatch<float, 64>(a, row0, rows, s) : pairs_dispatch<float, 128>(a, row0, rows, s);
}

hipError_t launch_bwd_dq(const BackwardArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((rows + 15) / 16));
  const bool half = a.dtype == BSA_BF16;
  if (a.d == 64) {
    if (half)
      hipLaunchKernelGGL((bwd_dq_kernel<64, true>), grid, dim3(256), 0, s, a.idx, a.dq_part, a.dq,
                         row0, rows, a.n, a.topk, a.causal, a.seqtab);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<64, false>), grid, dim3(256), 0, s, a.idx, a.dq_part, a.dq,
                         row0, rows, a.n, a.topk, a.causal, a.seqtab);
  } else {
    if (half)
      hipLaunchKernelGGL((bwd_dq_kernel<128, true>), grid, dim3(256), 0, s, a.idx, a.dq_part, a.dq,
                         row0, rows, a.n, a.topk, a.causal, a.seqtab);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<128, false>), grid, dim3(256), 0, s, a.idx, a.dq_part, a.dq,
                         row0, rows, a.n, a.topk, a.causal, a.seqtab);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkv(const BackwardArgs& a, int64_t row0, int64_t rows, hipStream_t s) {
  const Geom c(a, row0, rows);
  const dim3 grid(static_cast<unsigned>((c.bh1 - c.bh0 + 1) * c.nb));
  if (a.d == 64)
    hipLaunchKernelGGL(bwd_dkv_kernel<64>, grid, dim3(256), 0, s, a.dkv_part, a.ws.items, a.dk, a.dv, row0,
                       a.n, c.bh0, a.qsegs);
  else
    hipLaunchKernelGGL(bwd_dkv_kernel<128>, grid, dim3(256), 0, s, a.dkv_part, a.ws.items, a.dk, a.dv, row0,
                       a.n, c.bh0, a.qsegs);
  return hipGetLastError();
}

}  // namespace bsa
