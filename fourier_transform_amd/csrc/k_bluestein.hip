// Bluestein's chirp transform for C2C rows whose length is not a power of
// two: one kernel per batch of rows, each row going through two power-of-two
// transforms of length M >= 2n - 1 in registers and LDS, so a row is read
// from HBM once and written once.
//
// From jk = (j^2 + k^2 - (k - j)^2)/2:  y_k = c_k sum_j (x_j c_j) conj(c_{k-j})
// with c_j = e^{sign pi i j^2/n}, a circular convolution once the sequence
// x_j c_j is padded with zeros to M and conj(c) is wrapped around (entries
// M - j = entries j).  The convolution is the inverse transform of the
// product of the forward transforms; the forward transform of the wrapped
// chirp, divided by M, is a plan table (bhat) built on the host in f64, as
// are the chirps themselves (exponent j^2 reduced modulo 2n in integers).
// The lengths that are not powers of two are the route the GLSL
// dissertation ("High Performance Fourier Transforms on GPUs with GLSL",
// section 2.3) points to beyond radix-2 transforms.
#include "kernels.hpp"

namespace fftamd {

template <int M, int C>
__global__ __launch_bounds__(rows_threads(M) * C) void k_bluestein(BluesteinArgs a) {
  constexpr int E = rows_values(M);
  constexpr bool SPLIT = rows_split(M);
  constexpr int T = M / E;
  constexpr bool WL = T <= 64;  // every line inside one wavefront
  using L = RowLds<M, SPLIT, E>;
  static_assert(row_lds_bytes(M, C, SPLIT, E) <= kLdsBudgetBytes, "LDS budget");
  __shared__ lds_elem_t<SPLIT> lds[L::size(C)];
  lds_poison(lds);

  const int tid = threadIdx.x;
  const int line = tid / T, u = tid % T;
  const int64_t row = (int64_t)blockIdx.x * C + line;
  const bool valid = row < a.rows;
  const uint32_t n = (uint32_t)a.n;
  float2 v[E];
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const uint32_t j = (uint32_t)(u + T * m);
    v[m] = make_float2(0.f, 0.f);
    if (valid && j < n) v[m] = cmul(gload_nt(a.in + row * n, j), gload(a.pre, j));
  }
  run_stages<M, E, -1, WL, L, SPLIT>(v, lds, a.tw, u, line);
#pragma unroll
  for (int m = 0; m < E; ++m) v[m] = cmul(v[m], gload(a.bhat, (uint32_t)(u + T * m)));
  lds_sync<WL>();  // the first transform's last LDS reads precede the second's writes
  run_stages<M, E, +1, WL, L, SPLIT>(v, lds, a.tw, u, line);
  if (valid) {
    float2* dst = a.out + row * n;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const uint32_t j = (uint32_t)(u + T * m);
      if (j < n) gstore_nt(dst, j, cmul(v[m], gload(a.post, j)));
    }
  }
}

namespace {
template <int M>
struct BluesteinOp {
  static hipError_t run(const BluesteinArgs& a, hipStream_t st) {
    constexpr int C = rows_lines(M);
    uint32_t grid;
    hipError_t e = grid_of(a.rows, C, &grid);
    if (e != hipSuccess) return e;
    FFTAMD_LAUNCH((k_bluestein<M, C>), dim3(grid), dim3(rows_threads(M) * C), 0, st, a);
    return hipGetLastError();
  }
};
}  // namespace

hipError_t launch_bluestein(int m, const BluesteinArgs& a, hipStream_t st) {
  if (a.n < 2 || a.n > kMaxBluesteinLength || (int64_t)m < 2 * (int64_t)a.n - 1 || a.rows < 1)
    return hipErrorInvalidValue;
  return dispatch_pow2<BluesteinOp, 4, 2 * kMaxBluesteinLength>(m, a, st);
}

}  // namespace fftamd
