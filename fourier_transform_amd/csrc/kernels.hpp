// kernels.hpp -- transform kernels (templates over length and sign) and the
// per-length dispatch used by the launchers.
#pragma once

#include "launch.hpp"
#include "stockham.hpp"

namespace fftamd {

// ---------------------------------------------------------------------------
// workgroup shapes
// ---------------------------------------------------------------------------
constexpr int threads_per_line(int n) { return n / sched_e(n); }
constexpr int row_lds_bytes(int n, int c) { return c * (n + (n >> 4) + 1) * 8; }
constexpr int col_lds_bytes(int n, int c) { return (n * c + ((n * c) >> 4) + 1) * 8; }

// Row lanes: at least 256 threads per workgroup (several short rows share one).
constexpr int rows_per_wg(int n) {
  return threads_per_line(n) >= 256 ? 1 : 256 / threads_per_line(n);
}
// Column lanes: up to 16 adjacent lines (16 x 8 B = one 128 B segment per
// element index) within the thread and LDS limits.
constexpr int cols_per_wg(int n) {
  int c = 16;
  while (c > 1 && (c * threads_per_line(n) > kMaxThreads || col_lds_bytes(n, c) > kLdsBudgetBytes)) c /= 2;
  return c;
}
// Row lanes with a transposing store (four-step pass 2): as many lines as fit.
constexpr int tposed_rows_per_wg(int n) {
  int c = 16;
  while (c > 1 && (c * threads_per_line(n) > kMaxThreads || row_lds_bytes(n, c) > kLdsBudgetBytes)) c /= 2;
  return c;
}
// Real transforms: whole rows, >= 8 rows per workgroup so that m-major
// spectrum accesses form 64 B runs.
constexpr int real_rows_per_wg(int h) {
  int c = rows_per_wg(h) < 8 ? 8 : rows_per_wg(h);
  while (c > 1 && (c * threads_per_line(h) > kMaxThreads || row_lds_bytes(h, c) + c * 8 > kLdsBudgetBytes)) c /= 2;
  return c;
}

// ---------------------------------------------------------------------------
// C2C over contiguous rows
// ---------------------------------------------------------------------------
template <int N, int S, int C>
__global__ __launch_bounds__(threads_per_line(N) * C) void k_c2c_rows(RowsArgs a) {
  constexpr int E = sched_e(N);
  constexpr int T = N / E;
  constexpr bool WL = T <= 64;  // every line inside one wavefront
  using L = RowLds<N>;
  static_assert(row_lds_bytes(N, C) <= kLdsBudgetBytes, "LDS budget");
  __shared__ float2 lds[L::size(C)];

  const int tid = threadIdx.x;
  const int line = tid / T, u = tid % T;
  const int64_t row = (int64_t)blockIdx.x * C + line;
  const bool valid = row < a.rows;
  float2 v[E];
  if (valid) {
    const float2* src = a.in + row * N;
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = src[u + T * m];
    if (a.shift_mode) {
      const int par = a.shift_mode == 2 ? (int)(row & (a.rows_per_image - 1)) : 0;
#pragma unroll
      for (int m = 0; m < E; ++m)
        if ((par + u + T * m) & 1) v[m] = negate_bits(v[m]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = make_float2(0.f, 0.f);
  }
  run_stages<N, S, WL, L>(v, lds, a.tw, u, line);
  if (valid) {
    float2* dst = a.out + row * N;
#pragma unroll
    for (int m = 0; m < E; ++m) dst[u + T * m] = v[m];
  }
}

// ---------------------------------------------------------------------------
// C2C over columns of [images][N][nx] (2D column pass); in place allowed
// ---------------------------------------------------------------------------
template <int N, int S, int C>
__global__ __launch_bounds__(threads_per_line(N) * C) void k_c2c_cols(ColsArgs a) {
  constexpr int E = sched_e(N);
  constexpr int T = N / E;
  using L = ColLds<N, C>;
  static_assert(col_lds_bytes(N, C) <= kLdsBudgetBytes, "LDS budget");
  __shared__ float2 lds[L::size(C)];

  const int tid = threadIdx.x;
  const int line = tid % C, u = tid / C;
  const int64_t g = (int64_t)blockIdx.x * C + line;
  const bool valid = g < a.images * a.nx;
  const int64_t img = g / a.nx, col = g - img * a.nx;
  const float2* src = a.in + img * (int64_t)N * a.nx + col;
  float2* dst = a.out + img * (int64_t)N * a.nx + col;
  float2 v[E];
  if (valid) {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = src[(int64_t)(u + T * m) * a.nx];
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = make_float2(0.f, 0.f);
  }
  run_stages<N, S, false, L>(v, lds, a.tw, u, line);
  if (valid) {
#pragma unroll
    for (int m = 0; m < E; ++m) dst[(int64_t)(u + T * m) * a.nx] = v[m];
  }
}

// ---------------------------------------------------------------------------
// Real analysis (R2C) of rows of n = 2H reals: z_m = x_{2m} + i x_{2m+1},
// Z = forward FFT_H(z), X_k = Xe + e^{-2 pi i k/n} Xo with
// Xe = (Z_k + conj Z_{H-k})/2, Xo = -i (Z_k - conj Z_{H-k})/2 (Z_H = Z_0);
// turing-sphere fourier.ts, fftAnalysRealWGSL and its header comment.
// ---------------------------------------------------------------------------
template <int H, int C>
__global__ __launch_bounds__(threads_per_line(H) * C) void k_r2c(RealArgs a) {
  constexpr int E = sched_e(H);
  constexpr int T = H / E;
  constexpr bool WL = T <= 64;
  using L = RowLds<H>;
  static_assert(row_lds_bytes(H, C) <= kLdsBudgetBytes, "LDS budget");
  __shared__ float2 lds[L::size(C)];

  const int tid = threadIdx.x;
  const int line = tid / T, u = tid % T;
  const int64_t row = (int64_t)blockIdx.x * C + line;
  const bool valid = row < a.rows;
  float2 v[E];
  if (valid) {
    const float2* src = static_cast<const float2*>(a.in) + row * H;
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = src[u + T * m];
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = make_float2(0.f, 0.f);
  }
  run_stages<H, -1, WL, L>(v, lds, a.tw, u, line);
  __syncthreads();
#pragma unroll
  for (int m = 0; m < E; ++m) lds[L::at(line, u + T * m)] = v[m];
  __syncthreads();

  const int kout = a.mmax + 1;
  float2* out = static_cast<float2*>(a.out);
  for (int q = tid; q < C * kout; q += C * T) {
    int ln, k;
    if (a.mmajor) {
      ln = q % C;
      k = q / C;
    } else {
      ln = q / kout;
      k = q - ln * kout;
    }
    const int64_t r = (int64_t)blockIdx.x * C + ln;
    if (r >= a.rows) continue;
    const float2 zk = lds[L::at(ln, k & (H - 1))];
    const float2 zh = lds[L::at(ln, (H - k) & (H - 1))];
    const float2 xe = make_float2(0.5f * (zk.x + zh.x), 0.5f * (zk.y - zh.y));
    const float2 d = make_float2(0.5f * (zk.x - zh.x), 0.5f * (zk.y + zh.y));
    const float2 xo = make_float2(d.y, -d.x);
    const float2 X = cadd(xe, cmul(xo, a.rt[k]));
    out[a.mmajor ? (int64_t)k * a.rows + r : r * kout + k] = X;
  }
}

// ---------------------------------------------------------------------------
// Real synthesis (C2R): X from bins 0..mmax (X_0 = Re F_0, zero above mmax),
// Z_k = (X_k + conj X_{H-k}) + i e^{+2 pi i k/n} (X_k - conj X_{H-k}),
// z = inverse FFT_H(Z), x_{2m} = Re z_m, x_{2m+1} = Im z_m;
// turing-sphere fourier.ts, fftSynthRealWGSL and its header comment.
// ---------------------------------------------------------------------------
template <int H, int C>
__global__ __launch_bounds__(threads_per_line(H) * C) void k_c2r(RealArgs a) {
  constexpr int E = sched_e(H);
  constexpr int T = H / E;
  constexpr bool WL = T <= 64;
  using L = RowLds<H>;
  static_assert(row_lds_bytes(H, C) + C * 8 <= kLdsBudgetBytes, "LDS budget");
  __shared__ float2 lds[L::size(C)];
  __shared__ float2 nyq[C];

  const int tid = threadIdx.x;
  const int line = tid / T, u = tid % T;
  const int64_t row = (int64_t)blockIdx.x * C + line;
  const bool valid = row < a.rows;
  const int mmax = a.mmax;
  const int kin = mmax + 1;
  const float2* F = static_cast<const float2*>(a.in);

  // stage the spectra of the workgroup's rows in LDS (coalesced in either layout)
  for (int q = tid; q < C * kin; q += C * T) {
    int ln, k;
    if (a.mmajor) {
      ln = q % C;
      k = q / C;
    } else {
      ln = q / kin;
      k = q - ln * kin;
    }
    const int64_t r = (int64_t)blockIdx.x * C + ln;
    float2 val = make_float2(0.f, 0.f);
    if (r < a.rows) val = F[a.mmajor ? (int64_t)k * a.rows + r : r * kin + k];
    if (k < H)
      lds[L::at(ln, k)] = val;
    else
      nyq[ln] = val;
  }
  __syncthreads();

  float2 v[E];
  const float2 zero = make_float2(0.f, 0.f);
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int k = u + T * m;
    float2 xk;
    if (k == 0)
      xk = make_float2(lds[L::at(line, 0)].x, 0.f);
    else
      xk = k <= mmax ? lds[L::at(line, k)] : zero;
    const int kh = H - k;  // 1..H
    float2 xh;
    if (kh == H)
      xh = mmax >= H ? make_float2(nyq[line].x, 0.f) : zero;
    else
      xh = kh <= mmax ? lds[L::at(line, kh)] : zero;
    const float2 cj = cconj(xh);
    const float2 s = cadd(xk, cj);
    const float2 b = cmulc(csub(xk, cj), a.rt[k]);  // times e^{+2 pi i k/n}
    v[m] = make_float2(s.x - b.y, s.y + b.x);
  }
  __syncthreads();
  run_stages<H, +1, WL, L>(v, lds, a.tw, u, line);
  if (valid) {
    float2* dst = static_cast<float2*>(a.out) + row * H;
#pragma unroll
    for (int m = 0; m < E; ++m) dst[u + T * m] = v[m];
  }
}

// ---------------------------------------------------------------------------
// Four-step pass 1: column transforms of length N2 over stride n1, each
// output multiplied by W_n^{n1*k2}, stored in place of the column (to scratch)
// ---------------------------------------------------------------------------
template <int N2, int S, int C>
__global__ __launch_bounds__(threads_per_line(N2) * C) void k_fs_cols(FourStepArgs a) {
  constexpr int E = sched_e(N2);
  constexpr int T = N2 / E;
  using L = ColLds<N2, C>;
  static_assert(col_lds_bytes(N2, C) <= kLdsBudgetBytes, "LDS budget");
  __shared__ float2 lds[L::size(C)];

  const int tid = threadIdx.x;
  const int line = tid % C, u = tid / C;
  const int64_t g = (int64_t)blockIdx.x * C + line;
  const int64_t n1 = a.n1;
  const bool valid = g < a.batch * n1;
  const int64_t b = g / n1;
  const int c1 = (int)(g - b * n1);
  const int64_t base = b * n1 * N2 + c1;
  float2 v[E];
  if (valid) {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = a.in[base + (int64_t)(u + T * m) * n1];
    if (a.shift && (c1 & 1)) {  // element index c1 + n1*k has the parity of c1 (n1 even)
#pragma unroll
      for (int m = 0; m < E; ++m) v[m] = negate_bits(v[m]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = make_float2(0.f, 0.f);
  }
  run_stages<N2, S, false, L>(v, lds, a.tw, u, line);
  if (valid) {
    const uint32_t mask = (1u << a.bits) - 1u;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const uint32_t e = (uint32_t)c1 * (uint32_t)(u + T * m);
      const float2 w = cmul(a.thi[e >> a.bits], a.tlo[e & mask]);
      a.out[base + (int64_t)(u + T * m) * n1] = apply_tw<S>(v[m], w);
    }
  }
}

// ---------------------------------------------------------------------------
// Four-step pass 2: row transforms of length N1 over contiguous rows k2,
// element k1 stored at k2 + n2*k1 (through LDS so the stores are coalesced)
// ---------------------------------------------------------------------------
template <int N1, int S, int C>
__global__ __launch_bounds__(threads_per_line(N1) * C) void k_fs_rows(FourStepArgs a) {
  constexpr int E = sched_e(N1);
  constexpr int T = N1 / E;
  constexpr bool WL = T <= 64;
  using L = RowLds<N1>;
  static_assert(row_lds_bytes(N1, C) <= kLdsBudgetBytes, "LDS budget");
  __shared__ float2 lds[L::size(C)];

  const int tid = threadIdx.x;
  const int line = tid / T, u = tid % T;
  const int64_t n2 = a.n2;
  const int64_t lines = a.batch * n2;
  const int64_t g = (int64_t)blockIdx.x * C + line;
  const bool valid = g < lines;
  float2 v[E];
  if (valid) {
    const float2* src = a.in + g * N1;  // row k2 of transform b is at (b*n2 + k2)*N1
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = src[u + T * m];
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = make_float2(0.f, 0.f);
  }
  run_stages<N1, S, WL, L>(v, lds, a.tw, u, line);
  __syncthreads();
#pragma unroll
  for (int m = 0; m < E; ++m) lds[L::at(line, u + T * m)] = v[m];
  __syncthreads();
  for (int q = tid; q < C * N1; q += C * T) {
    const int ln = q % C, k1 = q / C;
    const int64_t gg = (int64_t)blockIdx.x * C + ln;
    if (gg >= lines) continue;
    const int64_t b = gg / n2;
    const int64_t k2 = gg - b * n2;
    a.out[b * n2 * N1 + (int64_t)k1 * n2 + k2] = lds[L::at(ln, k1)];
  }
}

// ---------------------------------------------------------------------------
// dispatch over power-of-two lengths
// ---------------------------------------------------------------------------
inline hipError_t grid_of(int64_t lines, int c, uint32_t* grid) {
  const int64_t g = (lines + c - 1) / c;
  if (g < 1 || g > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  *grid = (uint32_t)g;
  return hipSuccess;
}

template <template <int> class Op, int LO, int HI, class... Args>
hipError_t dispatch_pow2(int n, Args&&... args) {
  if constexpr (LO > HI) {
    return hipErrorInvalidValue;
  } else {
    if (n == LO) return Op<LO>::run(static_cast<Args&&>(args)...);
    return dispatch_pow2<Op, LO * 2, HI>(n, static_cast<Args&&>(args)...);
  }
}

}  // namespace fftamd
