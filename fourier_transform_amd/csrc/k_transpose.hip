// Tiled transpose of complex64 matrices, for 2D plans whose axes are not both
// powers of two: their column transform runs as row transforms of the
// transposed image (rows, transpose, rows, transpose back), since the
// any-length kernels read contiguous rows.
#include "kernels.hpp"

namespace fftamd {

namespace {
constexpr int kTile = 32;
constexpr int kTileRows = 8;  // 32 x 8 threads, 4 elements each

__global__ __launch_bounds__(kTile * kTileRows) void k_transpose(const float2* __restrict__ in,
                                                              float2* __restrict__ out, int64_t rows,
                                                              int64_t cols, int64_t tiles_c, int64_t rot) {
  __shared__ float2 tile[kTile][kTile + 1];
  lds_poison(tile);
  const int64_t img = blockIdx.y;
  const int64_t tr = (int64_t)blockIdx.x / tiles_c, tc = (int64_t)blockIdx.x % tiles_c;
  const int tx = threadIdx.x, ty = threadIdx.y;
  const float2* src = in + img * rows * cols;
  float2* dst = out + img * rows * cols;
#pragma unroll
  for (int i = 0; i < kTile; i += kTileRows) {
    const int64_t r = tr * kTile + ty + i, c = tc * kTile + tx;
    if (r < rows && c < cols) tile[ty + i][tx] = src[r * cols + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kTile; i += kTileRows) {
    const int64_t c = tc * kTile + ty + i, r = tr * kTile + tx;  // output row c, column r
    if (r < rows && c < cols) {
      int64_t e = c * rows + r + rot;
      if (e >= rows * cols) e -= rows * cols;
      dst[e] = tile[tx][ty + i];
    }
  }
}
}  // namespace

hipError_t launch_transpose(const float2* in, float2* out, int64_t rows, int64_t cols, int64_t images,
                            hipStream_t st, int64_t rot) {
  if (rows < 1 || cols < 1 || images < 1 || images > 65535 || rot < 0 || rot >= rows * cols)
    return hipErrorInvalidValue;
  const int64_t tiles_r = (rows + kTile - 1) / kTile, tiles_c = (cols + kTile - 1) / kTile;
  if (tiles_r * tiles_c > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  FFTAMD_LAUNCH(k_transpose, dim3((uint32_t)(tiles_r * tiles_c), (uint32_t)images),
                     dim3(kTile, kTileRows), 0, st, in, out, rows, cols, tiles_c, rot);
  return hipGetLastError();
}

}  // namespace fftamd
