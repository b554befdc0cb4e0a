// Instantiations and launcher of the contiguous-row C2C kernel.
#include "kernels.hpp"

namespace fftamd {
namespace {
template <int S>
struct RowsOp {
  template <int N>
  struct At {
    static hipError_t run(const RowsArgs& a, hipStream_t st) {
      constexpr int C = rows_lines(N);
      uint32_t grid;
      hipError_t e = grid_of(a.rows, C, &grid);
      if (e != hipSuccess) return e;
      FFTAMD_LAUNCH((k_c2c_rows<N, S, C>), dim3(grid), dim3(rows_threads(N) * C), 0, st, a);
      return hipGetLastError();
    }
  };
};
}  // namespace

hipError_t launch_c2c_rows(int n, int sign, const RowsArgs& a, hipStream_t st) {
  if (sign < 0) return dispatch_pow2<RowsOp<-1>::At, 2, kMaxSinglePass>(n, a, st);
  return dispatch_pow2<RowsOp<1>::At, 2, kMaxSinglePass>(n, a, st);
}
}  // namespace fftamd
