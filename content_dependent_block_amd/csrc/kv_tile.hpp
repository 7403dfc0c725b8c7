// kv_tile.hpp -- staging of one 64-key tile of K and V from HBM into LDS for
// the fine-attention kernels, split into a global->register half (issued
// early, so the loads overlap other work) and a register->LDS half.
//
// LDS layout:
//   K: [64 keys][D + pad], natural layout.  bf16: pad 16 elements (32 B); the
//      16-byte A-operand reads of 16 rows then run without bank conflicts on
//      gfx950 (with a 16-byte pad half the LDS cycles were conflicts).  fp32:
//      pad 4 elements.
//   V, bf16: transposed to [D][64 + 4 keys] so the A operand of
//      O^T = V^T P^T is two 8-byte reads per lane; two keys are packed per
//      32-bit LDS write.
//   V, fp32: natural [64 keys][D + 4].
// A workgroup of NTH threads (64, 128 or 256) moves one tile; every global
// load is 16 bytes and consecutive lanes read consecutive 16-byte pieces of a
// key row.
#pragma once

#include "bsa_device.hpp"

namespace bsa {

template <typename T, int D, int NTH = 256>
struct KvLayout {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int KPITCH = D + (kBf16 ? 16 : 4);       // elements per K row
  static constexpr int VROWS = kBf16 ? D : kTile;           // bf16: V^T rows are d
  static constexpr int VPITCH = kBf16 ? kTile + 4 : D + 4;  // elements per V row
  static constexpr int K_BYTES = kTile * KPITCH * sizeof(T);
  static constexpr int V_BYTES = VROWS * VPITCH * sizeof(T);
  static constexpr int BYTES = (K_BYTES + V_BYTES + 15) / 16 * 16;
  static constexpr int KCH = (kBf16 ? D / 32 : D / 16) * (256 / NTH);  // 16-byte K loads per thread
  static constexpr int VCH = (kBf16 ? D / 32 : D / 16) * (256 / NTH);  // 16-byte V loads per thread
};

template <typename T, int D, int NTH = 256>
struct KvRegs {
  uint4 kr[KvLayout<T, D, NTH>::KCH];
  uint4 vr[KvLayout<T, D, NTH>::VCH];
};

// Global loads of key tile `kt` (keys 64*kt .. 64*kt+63) of one head.  A
// tile with only `klim` < 64 keys in memory (the last tile of a sequence
// whose length is not a multiple of 64) reads key klim - 1 in place of the
// missing ones; the caller masks those keys.
template <typename T, int D, int NTH = 256>
__device__ __forceinline__ void kv_load(KvRegs<T, D, NTH>& r, const T* __restrict__ kb,
                                        const T* __restrict__ vb, int kt, int tid, int klim = kTile) {
  using L = KvLayout<T, D, NTH>;
  const int64_t key0 = static_cast<int64_t>(kt) * kTile;
  auto key = [&](int row) -> int64_t { return key0 + (row < klim ? row : klim - 1); };
  if constexpr (L::kBf16) {
#pragma unroll
    for (int u = 0; u < L::KCH; ++u) {
      const int c = tid + NTH * u, c8 = c % (D / 8), row = c / (D / 8);
      r.kr[u] = ld16(kb + key(row) * D + c8 * 8);
    }
#pragma unroll
    for (int u = 0; u < L::VCH / 2; ++u) {
      const int it = tid + NTH * u, c8 = it % (D / 8), p = it / (D / 8);
      r.vr[2 * u] = ld16(vb + key(2 * p) * D + c8 * 8);
      r.vr[2 * u + 1] = ld16(vb + key(2 * p + 1) * D + c8 * 8);
    }
  } else {
#pragma unroll
    for (int u = 0; u < L::KCH; ++u) {
      const int c = tid + NTH * u, c4 = c % (D / 4), row = c / (D / 4);
      r.kr[u] = ld16(kb + key(row) * D + c4 * 4);
      r.vr[u] = ld16(vb + key(row) * D + c4 * 4);
    }
  }
}

template <typename T, int D, int NTH = 256>
__device__ __forceinline__ void kv_store(const KvRegs<T, D, NTH>& r, T* ks, T* vs, int tid) {
  using L = KvLayout<T, D, NTH>;
  if constexpr (L::kBf16) {
#pragma unroll
    for (int u = 0; u < L::KCH; ++u) {
      const int c = tid + NTH * u, c8 = c % (D / 8), row = c / (D / 8);
      *reinterpret_cast<uint4*>(ks + row * L::KPITCH + c8 * 8) = r.kr[u];
    }
#pragma unroll
    for (int u = 0; u < L::VCH / 2; ++u) {
      const int it = tid + NTH * u, c8 = it % (D / 8), p = it / (D / 8);
      const uint32_t a[4] = {r.vr[2 * u].x, r.vr[2 * u].y, r.vr[2 * u].z, r.vr[2 * u].w};
      const uint32_t b[4] = {r.vr[2 * u + 1].x, r.vr[2 * u + 1].y, r.vr[2 * u + 1].z,
                             r.vr[2 * u + 1].w};
      uint32_t* dst = reinterpret_cast<uint32_t*>(vs + (c8 * 8) * L::VPITCH + 2 * p);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // d = c8*8 + 2e (low halves) and + 2e + 1 (high halves); keys 2p, 2p+1.
        dst[(2 * e) * (L::VPITCH / 2)] = (a[e] & 0xFFFFu) | (b[e] << 16);
        dst[(2 * e + 1) * (L::VPITCH / 2)] = (a[e] >> 16) | (b[e] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < L::KCH; ++u) {
      const int c = tid + NTH * u, c4 = c % (D / 4), row = c / (D / 4);
      *reinterpret_cast<uint4*>(ks + row * L::KPITCH + c4 * 4) = r.kr[u];
      *reinterpret_cast<uint4*>(vs + row * L::VPITCH + c4 * 4) = r.vr[u];
    }
  }
}

}  // namespace bsa
