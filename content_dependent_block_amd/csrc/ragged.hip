// ragged.hip -- row copies for sequences whose length is not a multiple of
// the 64-key block.  The library runs such sequences on copies in which every
// sequence starts on a block boundary and is padded with rows of `fill` to
// whole blocks (the padding keys masked in the kernels that could see them),
// and copies the rows that exist of the results back.  The block table
// (bsa_device.hpp) maps each block of the padded layout to the caller row its
// first row comes from.
#include "bsa_device.hpp"
#include "bsa_launch.hpp"

namespace bsa {
namespace {

// dst[h][r] = src[h][first caller row of block r / 64 + r % 64] for the rows
// that exist, fill for padding rows.
__global__ __launch_bounds__(256) void pad_rows_kernel(const uint32_t* __restrict__ src,
                                                       uint32_t* __restrict__ dst, int64_t slices,
                                                       int src_rows, int n_pad, int words, uint32_t fill,
                                                       const int4* __restrict__ seqtab) {
  const int64_t total = slices * n_pad * static_cast<int64_t>(words);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = e / words;
    const int w = static_cast<int>(e % words);
    const int64_t h = row / n_pad;
    const int r = static_cast<int>(row % n_pad);
    const int4 b = seqtab[r / kTile];
    const int t = r % kTile;
    dst[e] = t < b.z ? src[(h * src_rows + b.w + t) * words + w] : fill;
  }
}

// The inverse for the rows that exist: dst[h][caller row] = src[h][r].
__global__ __launch_bounds__(256) void unpad_rows_kernel(const uint32_t* __restrict__ src,
                                                         uint32_t* __restrict__ dst, int64_t slices,
                                                         int src_rows, int n_pad, int words,
                                                         const int4* __restrict__ seqtab) {
  const int64_t total = slices * n_pad * static_cast<int64_t>(words);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = e / words;
    const int w = static_cast<int>(e % words);
    const int64_t h = row / n_pad;
    const int r = static_cast<int>(row % n_pad);
    const int4 b = seqtab[r / kTile];
    const int t = r % kTile;
    if (t < b.z) dst[(h * src_rows + b.w + t) * words + w] = src[e];
  }
}

unsigned grid_for(int64_t total) {
  const int64_t g = (total + 255) / 256;
  return static_cast<unsigned>(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

}  // namespace

hipError_t launch_pad_rows(const void* src, void* dst, int64_t slices, int src_rows, int n_pad, int words,
                           uint32_t fill, const int4* seqtab, hipStream_t s) {
  hipLaunchKernelGGL(pad_rows_kernel, dim3(grid_for(slices * n_pad * static_cast<int64_t>(words))), dim3(256), 0,
                     s, static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), slices, src_rows, n_pad,
                     words, fill, seqtab);
  return hipGetLastError();
}

hipError_t launch_unpad_rows(const void* src, void* dst, int64_t slices, int src_rows, int n_pad, int words,
                             const int4* seqtab, hipStream_t s) {
  hipLaunchKernelGGL(unpad_rows_kernel, dim3(grid_for(slices * n_pad * static_cast<int64_t>(words))), dim3(256),
                     0, s, static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), slices, src_rows,
                     n_pad, words, seqtab);
  return hipGetLastError();
}

}  // namespace bsa
