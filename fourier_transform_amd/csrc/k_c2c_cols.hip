// Instantiations and launcher of the strided-column C2C kernel (2D column pass).
#include "kernels.hpp"

namespace fftamd {
namespace {
template <int S>
struct ColsOp {
  template <int N>
  struct At {
    static hipError_t run(const ColsArgs& a, hipStream_t st) {
      constexpr int C = tile_lines(N, false);
      uint32_t grid;
      hipError_t e = grid_of(a.images * a.nx, C, &grid);
      if (e != hipSuccess) return e;
      FFTAMD_LAUNCH((k_c2c_cols<N, S>), dim3(grid), dim3(C * (N / tile_e(N, false))), 0, st, a);
      return hipGetLastError();
    }
  };
};
}  // namespace

hipError_t launch_c2c_cols(int ny, int sign, const ColsArgs& a, hipStream_t st) {
  if (sign < 0) return dispatch_pow2<ColsOp<-1>::At, 2, kMaxSinglePass>(ny, a, st);
  return dispatch_pow2<ColsOp<1>::At, 2, kMaxSinglePass>(ny, a, st);
}
}  // namespace fftamd
