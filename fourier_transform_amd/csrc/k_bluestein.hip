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

// Values per thread: those of the row kernel, except for m = 32768 (lengths
// above 8192): 64 values and 512 threads, so that the line (128 KiB in the
// split exchange) fits one workgroup; 32 values and 1024 threads left 128
// VGPRs per lane and spilled 408 B.  One kernel instead of the three passes
// over m: per 512 MiB 10001 1891 -> 1279 us, 12289 1642 -> 1091, 16000 1216
// -> 897, 9001 2088 -> 1392, 16383 1366 -> 912.
constexpr int bluestein_values(int m) { return m > kMaxSinglePass ? kSplitValues : rows_values(m); }
template <int M, int C>
__global__ __launch_bounds__((M / bluestein_values(M)) * C) void k_bluestein(BluesteinArgs a) {
  constexpr int E = bluestein_values(M);
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
    if constexpr (E > 32) {  // bound the loads in flight (VGPR budget)
      if ((m & 15) == 15) __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  run_stages<M, E, -1, WL, L, SPLIT>(v, lds, a.tw, u, line);
  __builtin_amdgcn_sched_barrier(0);
  // opaque copies of the thread index for the later phases: the element
  // indices would otherwise stay live from the loads to the stores (at m =
  // 32768 they spilled 252 B per lane; 96 B of spills remain there)
  int ub = u;
  asm volatile("" : "+v"(ub));
#pragma unroll
  for (int m = 0; m < E; ++m) {
    v[m] = cmul(v[m], gload(a.bhat, (uint32_t)(ub + T * m)));
    if constexpr (E > 32) {
      if ((m & 15) == 15) __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  lds_sync<WL>();  // the first transform's last LDS reads precede the second's writes
  run_stages<M, E, +1, WL, L, SPLIT>(v, lds, a.tw, u, line);
  if (valid) {
    float2* dst = a.out + row * n;
    int us = u;
    asm volatile("" : "+v"(us));
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const uint32_t j = (uint32_t)(us + T * m);
      if (j < n) gstore_nt(dst, j, cmul(v[m], gload(a.post, j)));
    }
  }
}

namespace {
template <int M>
struct BluesteinOp {
  static hipError_t run(const BluesteinArgs& a, hipStream_t st) {
    constexpr int C = M > kMaxSinglePass ? 1 : rows_lines(M);  // one 32768-point line per workgroup
    uint32_t grid;
    hipError_t e = grid_of(a.rows, C, &grid);
    if (e != hipSuccess) return e;
    FFTAMD_LAUNCH((k_bluestein<M, C>), dim3(grid), dim3((M / bluestein_values(M)) * C), 0, st, a);
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
