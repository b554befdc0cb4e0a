// Instantiations and launcher of four-step pass 2 (lengths beyond one
// workgroup): row transforms over the block layout with a transposing store.
// Pass 1 is in k_fourstep_cols.hip.
#include "kernels.hpp"

namespace fftamd {
// sub-transform lengths of the four-step split of 2^15 .. 2^28
constexpr int kFourStepMin = 128;

namespace {
// The pass-2 kernel is specialised on the column count of the pass-1
// workgroups, which fixes the block layout of the scratch between them.  The
// split makes n1 = n2 or n1 = n2/2, so two variants cover each.
template <int S>
struct FsRowsOp {
  template <int N1>
  struct At {
    template <int BC>
    static hipError_t go(const FourStepArgs& a, hipStream_t st) {
      constexpr int C = tile_lines(N1, true);
      if ((a.batch * a.n2) % C != 0) return hipErrorInvalidValue;  // the kernel loads whole groups
      constexpr int threads = C * (N1 / tile_e(N1, true));
      uint32_t grid, resident = 0;
      hipError_t e = grid_of(a.batch * a.n2, C, &grid);
      if (e != hipSuccess) return e;
      if constexpr (fs_rows_persistent<N1>()) {
        // at most as many workgroups as run at once, each looping over tiles
        if ((e = resident_workgroups<k_fs_rows<N1, S, BC>>(threads, &resident)) != hipSuccess) return e;
        if (grid > resident) grid = resident;
      }
      FFTAMD_LAUNCH((k_fs_rows<N1, S, BC>), dim3(grid), dim3(threads), 0, st, a);
      return hipGetLastError();
    }
    static hipError_t run(const FourStepArgs& a, hipStream_t st) {
      if (a.n2 == N1) return go<tile_lines(N1, false)>(a, st);
      if (a.n2 == 2 * N1) return go<tile_lines(2 * N1, false)>(a, st);
      return hipErrorInvalidValue;
    }
  };
};
}  // namespace

hipError_t launch_fourstep_rows(int n1, int sign, const FourStepArgs& a, hipStream_t st) {
  if (sign < 0) return dispatch_pow2<FsRowsOp<-1>::At, kFourStepMin, kMaxSinglePass>(n1, a, st);
  return dispatch_pow2<FsRowsOp<1>::At, kFourStepMin, kMaxSinglePass>(n1, a, st);
}
}  // namespace fftamd
