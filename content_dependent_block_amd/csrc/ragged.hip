// ragged.hip -- row copies for sequences whose length is not a multiple of
// the 64-key block.  The library runs such a sequence on copies padded to
// whole blocks (the padding rows masked in the kernels that could see them)
// and copies the valid rows of the results back.
#include "bsa_device.hpp"
#include "bsa_launch.hpp"

namespace bsa {
namespace {

__global__ __launch_bounds__(256) void pad_rows_kernel(const uint32_t* __restrict__ src,
                                                       uint32_t* __restrict__ dst, int64_t bh, int n,
                                                       int n_pad, int words, uint32_t fill) {
  const int64_t total = bh * n_pad * static_cast<int64_t>(words);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = e / words;
    const int w = static_cast<int>(e % words);
    const int64_t h = row / n_pad;
    const int r = static_cast<int>(row % n_pad);
    dst[e] = r < n ? src[(h * n + r) * words + w] : fill;
  }
}

__global__ __launch_bounds__(256) void unpad_rows_kernel(const uint32_t* __restrict__ src,
                                                         uint32_t* __restrict__ dst, int64_t bh, int n,
                                                         int n_pad, int words) {
  const int64_t total = bh * n * static_cast<int64_t>(words);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = e / words;
    const int w = static_cast<int>(e % words);
    const int64_t h = row / n;
    const int r = static_cast<int>(row % n);
    dst[e] = src[(h * n_pad + r) * words + w];
  }
}

unsigned grid_for(int64_t total) {
  const int64_t g = (total + 255) / 256;
  return static_cast<unsigned>(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

}  // namespace

hipError_t launch_pad_rows(const void* src, void* dst, int64_t bh, int n, int n_pad, int words,
                           uint32_t fill, hipStream_t s) {
  hipLaunchKernelGGL(pad_rows_kernel, dim3(grid_for(bh * n_pad * static_cast<int64_t>(words))), dim3(256), 0, s,
                     static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), bh, n, n_pad, words, fill);
  return hipGetLastError();
}

hipError_t launch_unpad_rows(const void* src, void* dst, int64_t bh, int n, int n_pad, int words,
                             hipStream_t s) {
  hipLaunchKernelGGL(unpad_rows_kernel, dim3(grid_for(bh * n * static_cast<int64_t>(words))), dim3(256), 0, s,
                     static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), bh, n, n_pad, words);
  return hipGetLastError();
}

}  // namespace bsa
