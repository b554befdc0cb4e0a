// Instantiations and launchers of the real-input (R2C) and real-output (C2R)
// kernels: one complex transform of half length plus the Hermitian pack/unpack.
#include "kernels.hpp"

namespace fftamd {
namespace {
template <int H>
struct R2COp {
  static hipError_t run(const RealArgs& a, hipStream_t st) {
    constexpr int C = real_rows_per_wg(H);
    uint32_t grid;
    hipError_t e = grid_of(a.rows, C, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_r2c<H, C>), dim3(grid), dim3(threads_per_line(H) * C), 0, st, a);
    return hipGetLastError();
  }
};
template <int H>
struct C2ROp {
  static hipError_t run(const RealArgs& a, hipStream_t st) {
    constexpr int C = real_rows_per_wg(H);
    uint32_t grid;
    hipError_t e = grid_of(a.rows, C, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_c2r<H, C>), dim3(grid), dim3(threads_per_line(H) * C), 0, st, a);
    return hipGetLastError();
  }
};
template <int N>
struct R2CPairsOp {
  static hipError_t run(const RealArgs& a, hipStream_t st) {
    constexpr int C = real_rows_per_wg(N);
    uint32_t grid;
    hipError_t e = grid_of(a.rows / 2, C, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_r2c_pairs<N, C>), dim3(grid), dim3(threads_per_line(N) * C), 0, st, a);
    return hipGetLastError();
  }
};
template <int N>
struct C2RPairsOp {
  static hipError_t run(const RealArgs& a, hipStream_t st) {
    constexpr int C = real_rows_per_wg(N);
    uint32_t grid;
    hipError_t e = grid_of(a.rows / 2, C, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_c2r_pairs<N, C>), dim3(grid), dim3(threads_per_line(N) * C), 0, st, a);
    return hipGetLastError();
  }
};
}  // namespace

hipError_t launch_r2c_pairs(int n, const RealArgs& a, hipStream_t st) {
  return dispatch_pow2<R2CPairsOp, 4, kMaxSinglePass>(n, a, st);
}
hipError_t launch_c2r_pairs(int n, const RealArgs& a, hipStream_t st) {
  return dispatch_pow2<C2RPairsOp, 4, kMaxSinglePass>(n, a, st);
}

hipError_t launch_r2c(int h, const RealArgs& a, hipStream_t st) {
  return dispatch_pow2<R2COp, 2, kMaxSinglePass>(h, a, st);
}
hipError_t launch_c2r(int h, const RealArgs& a, hipStream_t st) {
  return dispatch_pow2<C2ROp, 2, kMaxSinglePass>(h, a, st);
}
}  // namespace fftamd
