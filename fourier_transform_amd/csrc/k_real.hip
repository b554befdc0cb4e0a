// Instantiations and launchers of the real-input (R2C) and real-output (C2R)
// kernels: one complex transform of half length plus the Hermitian pack/unpack.
#include "kernels.hpp"

namespace fftamd {
namespace {
// Rows per workgroup: real_rows_per_wg (>= 8 where a line is short, so that
// m-major spectrum accesses form 64 B runs), halved once or twice while that
// leaves fewer workgroups than the 256 CUs.  1024 rows of 2048 (8 per
// workgroup: 128 workgroups) measured r2c 8.1 -> 8.0 us and c2r 9.6 -> 8.7 us
// with 4.
constexpr int kFillWorkgroups = 256;
template <int C>
int real_split(int64_t rows) {
  int d = 1;
  while (d < 4 && C % (2 * d) == 0 && (rows + C / d - 1) / (C / d) < kFillWorkgroups) d *= 2;
  return d;
}
#define FFTAMD_REAL_OP(NAME, KERNEL, LEN, ROWS)                                                   \
  template <int LEN>                                                                              \
  struct NAME {                                                                                   \
    template <int C>                                                                              \
    static hipError_t go(const RealArgs& a, hipStream_t st) {                                     \
      uint32_t grid;                                                                              \
      hipError_t e = grid_of(ROWS, C, &grid);                                                     \
      if (e != hipSuccess) return e;                                                              \
      FFTAMD_LAUNCH((KERNEL<LEN, C>), dim3(grid), dim3(threads_per_line(LEN) * C), 0, st, a); \
      return hipGetLastError();                                                                   \
    }                                                                                             \
    static hipError_t run(const RealArgs& a, hipStream_t st) {                                    \
      constexpr int C = real_rows_per_wg(LEN);                                                    \
      const int d = real_split<C>(ROWS);                                                          \
      if constexpr (C % 4 == 0) {                                                                 \
        if (d == 4) return go<C / 4>(a, st);                                                      \
      }                                                                                           \
      if constexpr (C % 2 == 0) {                                                                 \
        if (d == 2) return go<C / 2>(a, st);                                                      \
      }                                                                                           \
      return go<C>(a, st);                                                                        \
    }                                                                                             \
  };
FFTAMD_REAL_OP(R2COp, k_r2c, H, a.rows)
FFTAMD_REAL_OP(C2ROp, k_c2r, H, a.rows)
FFTAMD_REAL_OP(R2CPairsOp, k_r2c_pairs, N, a.rows / 2)
FFTAMD_REAL_OP(C2RPairsOp, k_c2r_pairs, N, a.rows / 2)
#undef FFTAMD_REAL_OP
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
