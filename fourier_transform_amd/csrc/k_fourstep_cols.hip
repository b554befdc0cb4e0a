// Instantiations and launcher of four-step pass 1 (lengths beyond one
// workgroup): strided column transforms with the inter-pass twiddle fused
// into their block-layout store.  Pass 2 is in k_fourstep_rows.hip.
#include "kernels.hpp"

namespace fftamd {
// sub-transform lengths of the four-step split of 2^15 .. 2^28
constexpr int kFourStepMin = 128;

namespace {
// The pass-1 kernel is specialised on the row count of the pass-2 workgroups
// (and the reverse), which fixes the block layout of the scratch between
// them.  The split makes n1 = n2 or n1 = n2/2, so two variants cover each.
template <int S, bool HOOK>
struct FsColsOp {
  template <int N2>
  struct At {
    template <int BK>
    static hipError_t go(const FourStepArgs& a, hipStream_t st) {
      constexpr int C = tile_lines(N2, false);
      constexpr int threads = C * (N2 / tile_e(N2, false));
      if ((a.batch * a.n1) % C != 0) return hipErrorInvalidValue;  // the kernel loads whole groups
      uint32_t grid;
      hipError_t e = grid_of(a.batch * a.n1, C, &grid);
      if (e != hipSuccess) return e;
      FourStepArgs b = a;
      b.stagger = 0;
      if constexpr (fs_cols_persistent<N2, HOOK>()) {
        // at most as many workgroups as run at once, each looping over
        // tiles, half of them 7 us late
        const uint32_t tiles = grid;
        uint32_t resident = 0;
        if ((e = resident_workgroups<k_fs_cols<N2, S, BK, HOOK>>(threads, &resident)) != hipSuccess) return e;
        if (grid > resident) grid = resident;
        if ((e = stagger_ticks(7.0, tiles, grid, &b.stagger)) != hipSuccess) return e;
      }
      FFTAMD_LAUNCH((k_fs_cols<N2, S, BK, HOOK>), dim3(grid), dim3(threads), 0, st, b);
      return hipGetLastError();
    }
    static hipError_t run(const FourStepArgs& a, hipStream_t st) {
      if (a.n1 == N2) return go<tile_lines(N2, true)>(a, st);
      if (2 * a.n1 == N2) return go<tile_lines(N2 / 2, true)>(a, st);
      return hipErrorInvalidValue;
    }
  };
};
}  // namespace

hipError_t launch_fourstep_cols(int n2, int sign, const FourStepArgs& a, hipStream_t st, bool hook) {
  if (hook) {
    if (sign < 0) return dispatch_pow2<FsColsOp<-1, true>::At, kFourStepMin, kMaxSinglePass>(n2, a, st);
    return dispatch_pow2<FsColsOp<1, true>::At, kFourStepMin, kMaxSinglePass>(n2, a, st);
  }
  if (sign < 0) return dispatch_pow2<FsColsOp<-1, false>::At, kFourStepMin, kMaxSinglePass>(n2, a, st);
  return dispatch_pow2<FsColsOp<1, false>::At, kFourStepMin, kMaxSinglePass>(n2, a, st);
}
}  // namespace fftamd
