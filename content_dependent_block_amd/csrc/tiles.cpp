// tiles.cpp -- host-side builders of the static tile list consumed by
// bsa_forward_static (yayme/CUDA-kernel README: precompute the active
// (row tile, column tile) pairs on the CPU and let the kernel walk that list
// instead of scanning the mask; infra.bea.ai "Block-Sparse & Linear Attention
// Kernels", section 4: a compressed per-row list of active blocks as the mask
// representation).
//
// Format: CSR over 64-query tiles.  row_ptr[t] .. row_ptr[t+1] index the
// ascending key-tile ids of query tile t in col[], and rowmask[p][r] is the
// 64-bit visibility of the keys of listed tile p for query row r of the tile.
#include <cstdint>
#include <cstring>
#include <vector>

#include "bsa.h"

#define BSA_API extern "C" __attribute__((visibility("default")))

namespace {

// Shared driver: `row_bits(i, kt)` returns the 64-bit visibility of key tile
// kt for query row i.  The first pass counts the active tiles and fills
// row_ptr; the second (only when col is given) fills col and rowmask.
template <typename RowBits>
bsa_status build(int n, int tile, int32_t* row_ptr, int32_t* col, uint64_t* rowmask,
                 int64_t* nnz_inout, RowBits&& row_bits) {
  if (!row_ptr || !nnz_inout || n < 1) return BSA_ERR_INVALID_ARG;
  if (tile != 64 || n % 64 != 0) return BSA_ERR_UNSUPPORTED;
  const int nt = n / tile;
  auto active = [&](int qt, int kt) {
    for (int r = 0; r < tile; ++r)
      if (row_bits(qt * tile + r, kt) != 0) return true;
    return false;
  };
  int64_t total = 0;
  for (int qt = 0; qt < nt; ++qt) {
    row_ptr[qt] = static_cast<int32_t>(total);
    for (int kt = 0; kt < nt; ++kt) total += active(qt, kt);
  }
  row_ptr[nt] = static_cast<int32_t>(total);
  if (!col) {
    *nnz_inout = total;
    return BSA_OK;
  }
  if (*nnz_inout < total) return BSA_ERR_INVALID_ARG;
  std::vector<uint64_t> bits(static_cast<size_t>(tile));
  int64_t p = 0;
  for (int qt = 0; qt < nt; ++qt)
    for (int kt = 0; kt < nt; ++kt) {
      bool any = false;
      for (int r = 0; r < tile; ++r) {
        bits[r] = row_bits(qt * tile + r, kt);
        any = any || bits[r] != 0;
      }
      if (!any) continue;
      col[p] = kt;
      if (rowmask) std::memcpy(rowmask + p * tile, bits.data(), sizeof(uint64_t) * tile);
      ++p;
    }
  *nnz_inout = total;
  return BSA_OK;
}

}  // namespace

BSA_API bsa_status bsa_tiles_from_mask(const uint8_t* mask, int n, int tile, int32_t* row_ptr,
                                       int32_t* col, uint64_t* rowmask, int64_t* nnz_inout) {
  if (!mask) return BSA_ERR_INVALID_ARG;
  return build(n, tile, row_ptr, col, rowmask, nnz_inout, [&](int i, int kt) -> uint64_t {
    const uint8_t* m = mask + static_cast<int64_t>(i) * n + static_cast<int64_t>(kt) * 64;
    uint64_t b = 0;
    for (int c = 0; c < 64; ++c) b |= static_cast<uint64_t>(m[c] != 0) << c;
    return b;
  });
}

BSA_API bsa_status bsa_tiles_window_stride(int n, int window, int stride, int tile,
                                           int32_t* row_ptr, int32_t* col, uint64_t* rowmask,
                                           int64_t* nnz_inout) {
  if (window < 0 || stride < 1) return BSA_ERR_INVALID_ARG;
  return build(n, tile, row_ptr, col, rowmask, nnz_inout, [&](int i, int kt) -> uint64_t {
    uint64_t b = 0;
    const int j0 = kt * 64;
    // keys of the band [i - window, i + window] inside this tile
    int lo = i - window, hi = i + window;
    if (lo < j0) lo = j0;
    if (hi > j0 + 63) hi = j0 + 63;
    for (int j = lo; j <= hi; ++j) b |= 1ull << (j - j0);
    // global keys: multiples of stride inside this tile
    int first = (j0 + stride - 1) / stride * stride;
    for (int j = first; j < j0 + 64; j += stride) b |= 1ull << (j - j0);
    return b;
  });
}

BSA_API bsa_status bsa_tiles_validate(const int32_t* row_ptr, const int32_t* col, int64_t nnz,
                                      int n, int tile) {
  if (!row_ptr || nnz < 0 || n < 1 || tile < 1) return BSA_ERR_INVALID_ARG;
  if (tile != 64 || n % 64 != 0) return BSA_ERR_UNSUPPORTED;
  if (nnz > 0 && !col) return BSA_ERR_INVALID_ARG;
  const int nt = n / tile;
  if (row_ptr[0] != 0 || row_ptr[nt] != nnz) return BSA_ERR_INVALID_ARG;
  for (int t = 0; t < nt; ++t)
    if (row_ptr[t + 1] < row_ptr[t]) return BSA_ERR_INVALID_ARG;
  for (int64_t p = 0; p < nnz; ++p)
    if (col[p] < 0 || col[p] >= nt) return BSA_ERR_INVALID_ARG;
  return BSA_OK;
}
