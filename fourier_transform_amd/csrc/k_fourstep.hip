// Instantiations and launchers of the two four-step passes (lengths beyond one
// workgroup): strided column transforms with the inter-pass twiddle, then row
// transforms with a transposing store.
#include "kernels.hpp"

namespace fftamd {
// sub-transform lengths of the four-step split of 2^15 .. 2^28
constexpr int kFourStepMin = 128;

namespace {
template <int S>
struct FsColsOp {
  template <int N2>
  struct At {
    static hipError_t run(const FourStepArgs& a, hipStream_t st) {
      constexpr int C = tile_lines(N2, false);
      uint32_t grid;
      hipError_t e = grid_of(a.batch * a.n1, C, &grid);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((k_fs_cols<N2, S>), dim3(grid), dim3(C * (N2 / tile_e(N2, false))), 0, st, a);
      return hipGetLastError();
    }
  };
};
template <int S>
struct FsRowsOp {
  template <int N1>
  struct At {
    static hipError_t run(const FourStepArgs& a, hipStream_t st) {
      constexpr int C = tile_lines(N1, true);
      uint32_t grid;
      hipError_t e = grid_of(a.batch * a.n2, C, &grid);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((k_fs_rows<N1, S>), dim3(grid), dim3(C * (N1 / tile_e(N1, true))), 0, st, a);
      return hipGetLastError();
    }
  };
};
}  // namespace

hipError_t launch_fourstep_cols(int n2, int sign, const FourStepArgs& a, hipStream_t st) {
  if (sign < 0) return dispatch_pow2<FsColsOp<-1>::At, kFourStepMin, kMaxSinglePass>(n2, a, st);
  return dispatch_pow2<FsColsOp<1>::At, kFourStepMin, kMaxSinglePass>(n2, a, st);
}
hipError_t launch_fourstep_rows(int n1, int sign, const FourStepArgs& a, hipStream_t st) {
  if (sign < 0) return dispatch_pow2<FsRowsOp<-1>::At, kFourStepMin, kMaxSinglePass>(n1, a, st);
  return dispatch_pow2<FsRowsOp<1>::At, kFourStepMin, kMaxSinglePass>(n1, a, st);
}
}  // namespace fftamd
