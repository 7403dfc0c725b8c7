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
#include <cstdio>
#include <cstring>
#include <vector>

#include "bsa.h"

#define BSA_API extern "C" __attribute__((visibility("default")))

namespace {

// Shared driver: `row_bits(i, kt)` returns the 64-bit visibility of key tile
// kt for query row i (bits of keys at or past n clear).  The first pass
// counts the active tiles and fills row_ptr; the second (only when col is
// given) fills col and rowmask.  n need not be a multiple of the tile: the
// last query tile holds n mod 64 rows, the last key tile n mod 64 keys.
template <typename RowBits>
bsa_status build(int n, int tile, int32_t* row_ptr, int32_t* col, uint64_t* rowmask,
                 int64_t* nnz_inout, RowBits&& row_bits) {
  if (!row_ptr || !nnz_inout || n < 1) return BSA_ERR_INVALID_ARG;
  if (tile != 64) return BSA_ERR_UNSUPPORTED;
  const int nt = (n + tile - 1) / tile;
  auto rows_of = [&](int qt) { return qt * tile + tile <= n ? tile : n - qt * tile; };
  auto active = [&](int qt, int kt) {
    for (int r = 0; r < rows_of(qt); ++r)
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
        bits[r] = r < rows_of(qt) ? row_bits(qt * tile + r, kt) : 0ull;
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

namespace bsa {

// Every rule a tile list must satisfy for n rows and 64-wide tiles; on
// failure `why` (why_len bytes, may be NULL) says which.
bsa_status tiles_check(const int32_t* row_ptr, const int32_t* col, const uint64_t* rowmask, int64_t nnz,
                       int n, int tile, char* why, size_t why_len) {
  auto no = [&](bsa_status s, const char* fmt, long long a, long long b) {
    if (why && why_len) std::snprintf(why, why_len, fmt, a, b);
    return s;
  };
  if (n < 1) return no(BSA_ERR_INVALID_ARG, "n must be >= 1 (got %lld)%lld", n, 0);
  if (tile != 64) return no(BSA_ERR_UNSUPPORTED, "tile must be 64 (got %lld)%lld", tile, 0);
  if (!row_ptr) return no(BSA_ERR_INVALID_ARG, "row_ptr is NULL%lld%lld", 0, 0);
  if (nnz < 0) return no(BSA_ERR_INVALID_ARG, "nnz must be >= 0 (got %lld)%lld", nnz, 0);
  if (nnz > 0 && !col) return no(BSA_ERR_INVALID_ARG, "col is NULL with nnz = %lld%lld", nnz, 0);
  const int nt = (n + tile - 1) / tile;
  if (row_ptr[0] != 0) return no(BSA_ERR_INVALID_ARG, "row_ptr[0] = %lld, must be 0%lld", row_ptr[0], 0);
  if (row_ptr[nt] != nnz)
    return no(BSA_ERR_INVALID_ARG, "row_ptr[n_tiles] = %lld differs from nnz = %lld", row_ptr[nt], nnz);
  for (int t = 0; t < nt; ++t)
    if (row_ptr[t + 1] < row_ptr[t])
      return no(BSA_ERR_INVALID_ARG, "row_ptr decreases after query tile %lld (to %lld)", t, row_ptr[t + 1]);
  for (int t = 0; t < nt; ++t)
    for (int64_t p = row_ptr[t]; p < row_ptr[t + 1]; ++p) {
      if (col[p] < 0 || col[p] >= nt)
        return no(BSA_ERR_INVALID_ARG, "col[%lld] = %lld is not a key tile of the sequence", p, col[p]);
      if (p > row_ptr[t] && col[p] <= col[p - 1])
        return no(BSA_ERR_INVALID_ARG, "col[%lld] = %lld is not above the previous entry of its query tile", p,
                  col[p]);
    }
  const int klast = n - (nt - 1) * tile;
  if (rowmask && klast < tile) {
    const uint64_t past = ~((1ull << klast) - 1ull);  // keys at or past n in the last tile
    for (int64_t p = 0; p < nnz; ++p)
      if (col[p] == nt - 1)
        for (int r = 0; r < tile; ++r)
          if (rowmask[p * tile + r] & past)
            return no(BSA_ERR_INVALID_ARG, "rowmask of entry %lld row %lld shows a key past n", p, r);
  }
  return BSA_OK;
}

}  // namespace bsa

BSA_API bsa_status bsa_tiles_from_mask(const uint8_t* mask, int n, int tile, int32_t* row_ptr,
                                       int32_t* col, uint64_t* rowmask, int64_t* nnz_inout) {
  if (!mask) return BSA_ERR_INVALID_ARG;
  return build(n, tile, row_ptr, col, rowmask, nnz_inout, [&](int i, int kt) -> uint64_t {
    const uint8_t* m = mask + static_cast<int64_t>(i) * n;
    const int j0 = kt * 64, j1 = j0 + 64 < n ? j0 + 64 : n;
    uint64_t b = 0;
    for (int j = j0; j < j1; ++j) b |= static_cast<uint64_t>(m[j] != 0) << (j - j0);
    return b;
  });
}

BSA_API bsa_status bsa_tiles_window_stride(int n, int window, int stride, int tile,
                                           int32_t* row_ptr, int32_t* col, uint64_t* rowmask,
                                           int64_t* nnz_inout) {
  if (window < 0 || stride < 1) return BSA_ERR_INVALID_ARG;
  return build(n, tile, row_ptr, col, rowmask, nnz_inout, [&](int i, int kt) -> uint64_t {
    uint64_t b = 0;
    const int j0 = kt * 64, jend = (j0 + 63 < n - 1 ? j0 + 63 : n - 1);
    // keys of the band [i - window, i + window] inside this tile
    int lo = i - window, hi = i + window;
    if (lo < j0) lo = j0;
    if (hi > jend) hi = jend;
    for (int j = lo; j <= hi; ++j) b |= 1ull << (j - j0);
    // global keys: multiples of stride inside this tile
    int first = (j0 + stride - 1) / stride * stride;
    for (int j = first; j <= jend; j += stride) b |= 1ull << (j - j0);
    return b;
  });
}

BSA_API bsa_status bsa_tiles_validate(const int32_t* row_ptr, const int32_t* col, int64_t nnz,
                                      int n, int tile) {
  return bsa::tiles_check(row_ptr, col, nullptr, nnz, n, tile, nullptr, 0);
}
