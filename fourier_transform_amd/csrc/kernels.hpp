// kernels.hpp -- transform kernels (templates over length and sign) and the
// per-length dispatch used by the launchers.
#pragma once

#include <atomic>

#include "launch.hpp"
#include "shapes.hpp"
#include "stockham.hpp"

namespace fftamd {

template <bool SPLIT>
using lds_elem_t = typename std::conditional<SPLIT, float, float2>::type;

// Real transforms: whole rows, the largest rows-per-workgroup count (8 where
// a line is short) that fits the thread and LDS limits (80 KiB from lines of
// 2048 values), so that m-major spectrum accesses form 64 B runs on large
// batches.  The launchers
// (k_real.hip, real_split) run a half or a quarter of this count per
// workgroup while the full count would leave fewer workgroups than CUs
// (w4's 1024 rows of 2048: 4 rows per workgroup, 32 B runs).
constexpr int real_rows_per_wg(int h) {
  int c = rows_per_wg(h) < 8 ? 8 : rows_per_wg(h);
  // lines of 2048 values and more: at most 80 KiB of LDS, so that two
  // workgroups share a CU (one 8-row workgroup of 2048-point lines held a CU
  // alone): per 1 GiB of reals R2C / C2R at 4096 589 / 613 -> 497 / 554 us,
  // 8192 593 / 633 -> 506 / 551, 16384 644 / 687 -> 556 / 591
  while (c > 1 && (c * threads_per_line(h) > kMaxThreads || row_lds_bytes(h, c) + c * 8 > kLdsBudgetBytes ||
                   (h >= 2048 && row_lds_bytes(h, c) + c * 8 > 81920)))
    c /= 2;
  return c;
}

// ---------------------------------------------------------------------------
// C2C over contiguous rows
// ---------------------------------------------------------------------------
template <int N, int S, int C>
__global__ __launch_bounds__(rows_threads(N) * C) void k_c2c_rows(RowsArgs a) {
  constexpr int E = rows_values(N);
  constexpr bool SPLIT = rows_split(N);
  constexpr int T = N / E;
  constexpr bool WL = T <= 64;  // every line inside one wavefront
  // the wave's priority raised while it issues its row loads: per 512 MiB
  // 64 points 249 -> 237 us, 512 188 -> 177, 1024 191 -> 184, 2048 191 ->
  // 183, 16384 273 -> 265; no change at 4096, slower at 8192 (195 -> 207)
  constexpr bool LPRIO = N >= 64 && N != 4096 && N != 8192;
  using L = RowLds<N, SPLIT, E>;
  static_assert(row_lds_bytes(N, C, SPLIT, E) <= kLdsBudgetBytes, "LDS budget");
  // Rows of 4 to 32 points (one or two threads per row): a wavefront's loads
  // and stores would each touch up to 64 rows, so the workgroup's block of C
  // rows (contiguous) is read and written in order through LDS, rows SP =
  // N + 1 elements apart.  Per 512 MiB on MI355X: 8 points 370 -> 178 us,
  // 16 points 619 -> 230, 32 points 401 -> 252, 4 points 187 -> 169; 2 points
  // (163 -> 177) and 64 (249 -> 273) are faster unstaged.
  constexpr bool STAGE = T < 4 && N >= 4;
  constexpr int SP = N + 1;
  constexpr int LX = T > 1 ? L::size(C) : 1;  // lines of one thread exchange nothing
  constexpr int LE = STAGE && C * SP > LX ? C * SP : LX;
  __shared__ lds_elem_t<SPLIT> lds[LE];
  lds_poison(lds);

  const int tid = threadIdx.x;
  const int line = tid / T, u = tid % T;
  const int64_t row0 = (int64_t)blockIdx.x * C;
  const int64_t row = row0 + line;
  const bool valid = row < a.rows;
  const uint32_t off = (uint32_t)(line * N + u);
  constexpr uint32_t NT = (uint32_t)(C * T);
  const int64_t left = (a.rows - row0) * N;
  const uint32_t lim = left < (int64_t)C * N ? (uint32_t)left : (uint32_t)(C * N);
  float2 v[E];
  if constexpr (STAGE) {
    static_assert(!SPLIT, "staged rows use the complex exchange");
    const float2* src = a.in + row0 * N;
    if constexpr (LPRIO) __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const uint32_t i = (uint32_t)tid + NT * m;
      const float2 x = i < lim ? gload_nt(src, i) : make_float2(0.f, 0.f);
      lds[(i / N) * SP + i % N] = x;
    }
    if constexpr (LPRIO) __builtin_amdgcn_s_setprio(0);
    lds_barrier();
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = lds[line * SP + u + T * m];
    if (valid && a.shift_mode) {
      const int par = a.shift_mode == 2 ? (int)(row & (a.rows_per_image - 1)) : 0;
#pragma unroll
      for (int m = 0; m < E; ++m)
        if ((par + u + T * m) & 1) v[m] = negate_bits(v[m]);
    }
    lds_barrier();  // the stages reuse the buffer
  } else if (valid) {
    const float2* src = a.in + row0 * N;
    if constexpr (LPRIO) __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = gload_nt(src + T * m, off);
    if constexpr (LPRIO) __builtin_amdgcn_s_setprio(0);
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
  run_stages<N, E, S, WL, L, SPLIT>(v, lds, a.tw, u, line);
  if constexpr (STAGE) {
    lds_barrier();  // the last stage's exchange reads are done
#pragma unroll
    for (int m = 0; m < E; ++m) lds[line * SP + u + T * m] = v[m];
    lds_barrier();
    float2* dst = a.out + row0 * N;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const uint32_t i = (uint32_t)tid + NT * m;
      if (i < lim) {
        const float2 x = lds[(i / N) * SP + i % N];
        if (a.stream_store)
          gstore_nt(dst, i, x);
        else
          gstore(dst, i, x);
      }
    }
  } else if (valid) {
    float2* dst = a.out + row0 * N;
    if (a.stream_store) {
#pragma unroll
      for (int m = 0; m < E; ++m) gstore_nt(dst + T * m, off, v[m]);
    } else {
#pragma unroll
      for (int m = 0; m < E; ++m) gstore(dst, off + T * m, v[m]);
    }
  }
}

// ---------------------------------------------------------------------------
// C2C over columns of [images][N][nx] (2D column pass); in place allowed.
// C adjacent columns per workgroup, consecutive threads on consecutive columns.
// ---------------------------------------------------------------------------
template <int N, int S>
__global__ __launch_bounds__(tile_lines(N, false) * (N / tile_e(N, false))) void k_c2c_cols(ColsArgs a) {
  constexpr int E = tile_e(N, false);
  constexpr bool SPLIT = tile_split(N, false);
  constexpr int C = tile_lines(N, false);
  constexpr int T = N / E;
  using L = ColLds<N, C, SPLIT>;
  static_assert(L::size(C) * sizeof(lds_elem_t<SPLIT>) <= kLdsBudgetBytes, "LDS budget");
  __shared__ lds_elem_t<SPLIT> lds[L::size(C)];
  lds_poison(lds);

  const int tid = threadIdx.x;
  const int line = tid % C, u = tid / C;
  // the group's first column sets a uniform base; every element is then a
  // 32-bit offset from it (a group spans several images only when nx < C)
  const int64_t g0 = (int64_t)xcd_grouped_block(blockIdx.x, gridDim.x) * C;
  const bool valid = g0 + line < a.images * a.nx;
  const uint32_t nx = (uint32_t)a.nx;
  const int64_t img0 = g0 / nx;
  const uint32_t col0 = (uint32_t)(g0 - img0 * nx);
  const int64_t base = img0 * (int64_t)N * nx + col0;
  const uint32_t rel = (uint32_t)line + col0;
  const uint32_t off = (rel / nx) * (uint32_t)N * nx + rel % nx - col0 + (uint32_t)u * nx;
  const uint32_t step = (uint32_t)T * nx;
  float2 v[E];
  if (valid) {
    const float2* src = a.in + base;
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = gload(src, off + step * m);
    if (a.shift) {  // slot m holds row u + T*m: (-1)^row
#pragma unroll
      for (int m = 0; m < E; ++m)
        if ((u + T * m) & 1) v[m] = negate_bits(v[m]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = make_float2(0.f, 0.f);
  }
  run_stages<N, E, S, false, L, SPLIT>(v, lds, a.tw, u, line);
  if (valid) {
    float2* dst = a.out + base;
#pragma unroll
    for (int m = 0; m < E; ++m) gstore(dst, off + step * m, v[m]);
  }
}

// q / d for q * d < 2^32 by a multiply-high with floor((2^32 - 1) / d) + 1
struct FastDiv {
  uint32_t d, magic;
  __device__ explicit FastDiv(uint32_t d_) : d(d_), magic(0xffffffffu / d_ + 1u) {}
  __device__ __forceinline__ uint32_t div(uint32_t q) const { return d == 1 ? q : __umulhi(q, magic); }
};

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
  lds_poison(lds);

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
  run_stages<H, E, -1, WL, L, false>(v, lds, a.tw, u, line);
  lds_barrier();
  static_for<0, E>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    lds[L::template at_k<T * m>(line, u)] = v[m];
  });
  lds_barrier();

  const int kout = a.mmax + 1;
  const FastDiv dk((uint32_t)kout);
  float2* out = static_cast<float2*>(a.out);
  for (int q = tid; q < C * kout; q += C * T) {
    int ln, k;
    if (a.mmajor) {
      ln = q % C;
      k = q / C;
    } else {
      ln = (int)dk.div((uint32_t)q);
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
  lds_poison(lds, nyq);

  const int tid = threadIdx.x;
  const int line = tid / T, u = tid % T;
  const int64_t row = (int64_t)blockIdx.x * C + line;
  const bool valid = row < a.rows;
  const int mmax = a.mmax;
  const int kin = mmax + 1;
  const float2* F = static_cast<const float2*>(a.in);

  // stage the spectra of the workgroup's rows in LDS (coalesced in either
  // layout), U loads in flight per thread before their LDS stores (one load
  // at a time, each waited for before its store, took 1.4-1.7x as long: per
  // 1 GiB of reals 2048 746 -> 524 us, 256 663 -> 469, 8 1667 -> 998)
  const FastDiv dk((uint32_t)kin);
  const int tot = C * kin;
  constexpr int U = 8;
  for (int q0 = tid; q0 < tot; q0 += U * C * T) {
    float2 val[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int q = q0 + i * C * T;
      const int ln = a.mmajor ? q % C : (int)dk.div((uint32_t)q);
      const int k = a.mmajor ? q / C : q - ln * kin;
      const int64_t r = (int64_t)blockIdx.x * C + ln;
      val[i] = make_float2(0.f, 0.f);
      if (q < tot && r < a.rows) val[i] = F[a.mmajor ? (int64_t)k * a.rows + r : r * kin + k];
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int q = q0 + i * C * T;
      if (q < tot) {
        const int ln = a.mmajor ? q % C : (int)dk.div((uint32_t)q);
        const int k = a.mmajor ? q / C : q - ln * kin;
        if (k < H)
          lds[L::at(ln, k)] = val[i];
        else
          nyq[ln] = val[i];
      }
    }
  }
  lds_barrier();

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
  lds_barrier();
  run_stages<H, E, +1, WL, L, false>(v, lds, a.tw, u, line);
  // rows of 32 reals (16-value lines of one thread) are stored in order
  // through LDS: per 1 GiB of reals 495 -> 402 us; the shorter ones were
  // slower that way (8 reals 997 -> 1093 us, 16 1207 -> 1308)
  constexpr bool STG = T == 1 && H == 16;
  if constexpr (STG) {
#pragma unroll
    for (int m = 0; m < E; ++m) lds[L::at(line, m)] = v[m];
    lds_barrier();
    float2* dst = static_cast<float2*>(a.out) + (int64_t)blockIdx.x * C * H;
    const int64_t left = (a.rows - (int64_t)blockIdx.x * C) * H;
    const int lim = left < C * H ? (int)left : C * H;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const int i = tid + C * m;
      if (i < lim) dst[i] = lds[L::at(i / H, i % H)];
    }
  } else if (valid) {
    float2* dst = static_cast<float2*>(a.out) + row * H;
#pragma unroll
    for (int m = 0; m < E; ++m) dst[u + T * m] = v[m];
  }
}

// ---------------------------------------------------------------------------
// Two real rows in one complex transform ("High Performance Fourier
// Transforms on GPUs with GLSL", section 2.6, Equations 17-18): rows 2p and
// 2p+1 become the real and imaginary parts of y, Y = FFT_N(y), and
// X1(k) = (Y(k) + conj Y(N-k))/2, X2(k) = (Y(k) - conj Y(N-k))/(2i).
// (Equation 18 is printed garbled; this is its reading, consistent with the
// Xe/Xo split of the WGSL Fourier-stage source.)
// ---------------------------------------------------------------------------
template <int N, int C>
__global__ __launch_bounds__(threads_per_line(N) * C) void k_r2c_pairs(RealArgs a) {
  constexpr int E = real_values(N);
  constexpr int T = N / E;
  constexpr bool WL = T <= 64;
  using L = RowLds<N>;
  static_assert(row_lds_bytes(N, C) <= kLdsBudgetBytes, "LDS budget");
  __shared__ float2 lds[L::size(C)];
  lds_poison(lds);

  const int tid = threadIdx.x;
  const int line = tid / T, u = tid % T;
  const int64_t pairs = a.rows / 2;
  const int64_t pair = (int64_t)blockIdx.x * C + line;
  float2 v[E];
  if (pair < pairs) {
    const float* x1 = static_cast<const float*>(a.in) + 2 * pair * N;
    const float* x2 = x1 + N;
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = make_float2(x1[u + T * m], x2[u + T * m]);
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = make_float2(0.f, 0.f);
  }
  run_stages<N, E, -1, WL, L, false>(v, lds, a.tw, u, line);
  lds_barrier();
  static_for<0, E>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    lds[L::template at_k<T * m>(line, u)] = v[m];
  });
  lds_barrier();

  // outputs: (line, row of the pair, bin k); consecutive threads take
  // consecutive bins (row-major) or consecutive rows (m-major)
  const int kout = a.mmax + 1;
  const FastDiv dk((uint32_t)kout);
  float2* out = static_cast<float2*>(a.out);
  for (int q = tid; q < C * 2 * kout; q += C * T) {
    int ln, which, k;
    if (a.mmajor) {
      const int r = q % (2 * C);
      ln = r >> 1;
      which = r & 1;
      k = q / (2 * C);
    } else {
      const int r = (int)dk.div((uint32_t)q);
      ln = r >> 1;
      which = r & 1;
      k = q - r * kout;
    }
    const int64_t p = (int64_t)blockIdx.x * C + ln;
    if (p >= pairs) continue;
    const float2 yk = lds[L::at(ln, k)];
    const float2 ym = lds[L::at(ln, (N - k) & (N - 1))];
    float2 X;
    if (which == 0) {
      X = make_float2(0.5f * (yk.x + ym.x), 0.5f * (yk.y - ym.y));   // (Y(k) + conj Y(N-k)) / 2
    } else {
      const float dr = yk.x - ym.x, di = yk.y + ym.y;                 // Y(k) - conj Y(N-k)
      X = make_float2(0.5f * di, -0.5f * dr);                         // divided by 2i
    }
    const int64_t row = 2 * p + which;
    out[a.mmajor ? (int64_t)k * a.rows + row : row * kout + k] = X;
  }
}

template <int N, int C>
__global__ __launch_bounds__(threads_per_line(N) * C) void k_c2r_pairs(RealArgs a) {
  constexpr int E = real_values(N);
  constexpr int T = N / E;
  constexpr int H = N / 2;
  constexpr bool WL = T <= 64;
  using L = RowLds<N>;
  static_assert(row_lds_bytes(N, C) + 2 * C * 8 <= kLdsBudgetBytes, "LDS budget");
  __shared__ float2 lds[L::size(C)];
  __shared__ float2 nyq[2 * C];
  lds_poison(lds, nyq);

  const int tid = threadIdx.x;
  const int line = tid / T, u = tid % T;
  const int64_t pairs = a.rows / 2;
  const int64_t pair = (int64_t)blockIdx.x * C + line;
  const int mmax = a.mmax;
  const int kin = mmax + 1;
  const float2* F = static_cast<const float2*>(a.in);

  // stage both spectra: row 2p at [0, H), row 2p+1 at [H, N); bin H apart;
  // U loads in flight per thread before their LDS stores
  const FastDiv dk((uint32_t)kin);
  const int tot = C * 2 * kin;
  constexpr int U = 8;
  auto decode = [&](int q, int& ln, int& which, int& k) {
    const int r = a.mmajor ? q % (2 * C) : (int)dk.div((uint32_t)q);
    ln = r >> 1;
    which = r & 1;
    k = a.mmajor ? q / (2 * C) : q - r * kin;
  };
  for (int q0 = tid; q0 < tot; q0 += U * C * T) {
    float2 val[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int q = q0 + i * C * T;
      int ln, which, k;
      decode(q, ln, which, k);
      const int64_t p = (int64_t)blockIdx.x * C + ln;
      const int64_t row = 2 * p + which;
      val[i] = make_float2(0.f, 0.f);
      if (q < tot && p < pairs) val[i] = F[a.mmajor ? (int64_t)k * a.rows + row : row * kin + k];
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int q = q0 + i * C * T;
      if (q < tot) {
        int ln, which, k;
        decode(q, ln, which, k);
        if (k < H)
          lds[L::at(ln, which * H + k)] = val[i];
        else
          nyq[2 * ln + which] = val[i];
      }
    }
  }
  lds_barrier();

  // Y(k) = X1(k) + i X2(k) with each X Hermitian from its bins 0..mmax
  float2 v[E];
  const float2 zero = make_float2(0.f, 0.f);
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int k = u + T * m;
    float2 x[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float2 t;
      // value selects (a select between an LDS and a private lvalue put
      // the zero in scratch)
      if (k == 0) {
        t = make_float2(lds[L::at(line, w * H)].x, 0.f);
      } else if (k == H) {
        t = make_float2(mmax >= H ? nyq[2 * line + w].x : 0.f, 0.f);
      } else if (k < H) {
        const float2 l = lds[L::at(line, w * H + k)];
        t = k <= mmax ? l : zero;
      } else {
        const float2 l = cconj(lds[L::at(line, w * H + N - k)]);
        t = N - k <= mmax ? l : zero;
      }
      x[w] = t;
    }
    v[m] = make_float2(x[0].x - x[1].y, x[0].y + x[1].x);
  }
  lds_barrier();
  run_stages<N, E, +1, WL, L, false>(v, lds, a.tw, u, line);
  if (pair < pairs) {
    float* y1 = static_cast<float*>(a.out) + 2 * pair * N;
    float* y2 = y1 + N;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      y1[u + T * m] = v[m].x;
      y2[u + T * m] = v[m].y;
    }
  }
}

// ---------------------------------------------------------------------------
// Intermediate layout of the four-step split (plan scratch, one transform
// after the other).  Value (k2, c1) -- bin k2 of the column transform of
// column c1 -- sits in a block of BK x BC values:
//   ((k2 / BK) * (n1 / BC) + c1 / BC) * BK * BC + (k2 % BK) * BC + c1 % BC
// BC is the number of columns a pass-1 workgroup transforms and BK the number
// of rows a pass-2 workgroup transforms, so pass 1 stores whole blocks and
// pass 2 reads whole blocks: both sides of the scratch are contiguous runs,
// and only the caller's input (pass 1) and output (pass 2) are strided.
// ---------------------------------------------------------------------------
template <int BK, int BC>
__device__ __forceinline__ uint32_t fs_block_index(uint32_t k2, uint32_t c1, uint32_t n1) {
  return ((k2 / BK) * (n1 / BC) + c1 / BC) * (BK * BC) + (k2 % BK) * BC + c1 % BC;
}

// Stage 1 of the four-step passes reads its twiddles from an LDS copy of its
// part of the table when that fits beside the exchange buffers: R - 1 factors
// per butterfly from a 2-level L2 path otherwise, with two workgroups' worth
// of latency to hide at one workgroup per CU.
template <int N, int E>
constexpr int fs_tw1_elems() {
  return sched_stages(N, E) >= 2 ? sched_tw_off(N, E, 2) - sched_tw_off(N, E, 1) : 0;
}
template <int N, int E, int NT, int TQ>
__device__ __forceinline__ void fs_fetch_tw1(float2* tq, const float2* __restrict__ tw, int tid) {
  constexpr int O1 = sched_tw_off(N, E, 1);
#pragma unroll
  for (int i = 0; i < TQ; ++i) {  // clamped rather than skipped: every wave issues the same loads
    const int q = tid + NT * i;
    tq[i] = gload(tw, (uint32_t)(O1 + (q < fs_tw1_elems<N, E>() ? q : fs_tw1_elems<N, E>() - 1)));
  }
}
template <int N, int E, int NT, int TQ>
__device__ __forceinline__ void fs_store_tw1(float2* twl, const float2* tq, int tid) {
#pragma unroll
  for (int i = 0; i < TQ; ++i) {
    const int q = tid + NT * i;
    if (q < fs_tw1_elems<N, E>()) twl[q] = tq[i];
  }
}

// ---------------------------------------------------------------------------
// Four-step pass 1: column transforms of length N2 over stride n1, each
// output multiplied by W_n^{n1*k2}, stored to scratch in the block layout
// above (BK: rows per pass-2 workgroup)
//
// Tiles of 64 values per thread (N2 >= 2048) are persistent, with a
// staggered start (stagger_start): 2^22 x 32 pass 1 456 -> 439-441 us per
// launch with half of the workgroups 6-8 us late (4: 443, 10: 443, 12: 453;
// persistent without the stagger: no change).  The smaller tiles, and the
// hooked pass of the chirp transform (its extra live values spill in the
// loop), launch one workgroup per tile and run the loop once.
// ---------------------------------------------------------------------------
template <int N2, bool HOOK>
constexpr bool fs_cols_persistent() {
  return !HOOK && tile_e(N2, false) == kSplitValues;
}
template <int N2, int S, int BK, bool HOOK>
__global__ __launch_bounds__(tile_lines(N2, false) * (N2 / tile_e(N2, false)))
__attribute__((amdgpu_waves_per_eu(fs_waves(N2)))) void k_fs_cols(FourStepArgs a) {
  constexpr int E = tile_e(N2, false);
  constexpr bool SPLIT = tile_split(N2, false);
  constexpr int C = tile_lines(N2, false);
  constexpr int T = N2 / E;
  using L = ColLds<N2, C, SPLIT>;
  constexpr int FP = E + 1;  // row pitch of the factor table (spreads the lines over the banks)
  static_assert(L::size(C) * sizeof(lds_elem_t<SPLIT>) + C * FP * sizeof(float2) <= kLdsBudgetBytes,
                "LDS budget");
  // the stages' exchange barriers order the factor-table writes before the reads
  static_assert(sched_stages(N2, E) >= 2, "pass 1 needs at least one LDS exchange");
  constexpr int TW1 = fs_tw1_elems<N2, E>();
  constexpr bool LTW = L::size(C) * sizeof(lds_elem_t<SPLIT>) + (C * FP + TW1) * sizeof(float2) <= kLdsBudgetBytes;
  __shared__ lds_elem_t<SPLIT> lds[L::size(C)];
  __shared__ float2 ftab[C * FP];
  __shared__ float2 twl[LTW ? TW1 : 1];
  lds_poison(lds, ftab, twl);

  constexpr bool PERSIST = fs_cols_persistent<N2, HOOK>();
  constexpr int NT = C * T;
  // stage-1 twiddles: copied to LDS once per workgroup when persistent; else
  // fetched with the small loads below and stored after the line's loads.
  // Stage 0's exchange barriers order the copy before its reads.
  constexpr int TQ = LTW ? (TW1 + NT - 1) / NT : 1;
  if constexpr (LTW && PERSIST) {
    float2 tq[TQ];
    fs_fetch_tw1<N2, E, NT, TQ>(tq, a.tw, threadIdx.x);
    fs_store_tw1<N2, E, NT, TQ>(twl, tq, threadIdx.x);
  }
  if constexpr (PERSIST) stagger_start(a.stagger);
  const uint32_t ntiles = (uint32_t)(a.batch * a.n1 / C);  // whole groups (checked by the launcher)
  for (uint32_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
  // a per-tile opaque copy of the thread index: what derives from it is
  // recomputed per tile rather than kept live across the loop (spills)
  int tid = threadIdx.x;
  if constexpr (PERSIST) asm volatile("" : "+v"(tid));
  const int line = tid % C, u = tid / C;
  // n1 >= 128 > C: the group's columns belong to one transform b.  n1 is a
  // power of two: shifts, not a 64-bit division (whose reciprocal the
  // compiler would keep live across the tile loop)
  const int64_t g0 = (int64_t)xcd_grouped_block(tile, ntiles) * C;
  const uint32_t n1 = (uint32_t)a.n1;
  const bool valid = g0 + line < a.batch * (int64_t)n1;
  const uint32_t n1_log2 = (uint32_t)__builtin_ctz(n1);
  const int64_t b = g0 >> n1_log2;
  const uint32_t c1 = (uint32_t)(g0 & (int64_t)(n1 - 1)) + line;
  const int64_t base = (HOOK ? b * a.in_stride : b * (int64_t)n1 * N2) + (c1 - line);
  const uint32_t off = (uint32_t)line + (uint32_t)u * n1;
  const uint32_t step = (uint32_t)T * n1;
  // Inter-pass twiddle W_n^{c1*k2} with k2 = u + T*m, split as
  // W_n^{c1*u} * W_n^{c1*T*m}: the first factor is one per thread, the
  // second a table of C x E values per workgroup kept in LDS, so no value
  // needs a scattered table lookup per element.  Each factor is read as
  // thi[e >> bits] * tlo[e & mask] (both exponents stay below n).
  const uint32_t mask = (1u << a.bits) - 1u;
  const uint32_t c0 = c1 - line;
  // The small loads (factor table, this thread's factor, the stage-1
  // twiddles) are issued first and consumed only after the line's loads have
  // been issued: loads complete in issue order, so waiting for them then does
  // not wait for the line.
  constexpr int FQ = (C * E + NT - 1) / NT;
  float2 fh[FQ], fl[FQ];
#pragma unroll
  for (int i = 0; i < FQ; ++i) {
    const int q = tid + NT * i;
    if ((C * E) % NT == 0 || q < C * E) {
      const uint32_t e = (c0 + (uint32_t)(q / E)) * (uint32_t)(T * (q % E));
      fh[i] = gload(a.thi, e >> a.bits);
      fl[i] = gload(a.tlo, e & mask);
    }
  }
  float2 tq[TQ];
  if constexpr (LTW && !PERSIST) fs_fetch_tw1<N2, E, NT, TQ>(tq, a.tw, tid);
  __builtin_amdgcn_sched_barrier(0);
  float2 v[E];
  if (valid && HOOK) {
    // element j = c1 + n1*k2 of a row of in_len values (zero beyond), times pre[j]
    const float2* src = a.in + base;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const uint32_t j = c0 + off + step * m;
      v[m] = make_float2(0.f, 0.f);
      if (j < (uint32_t)a.in_len) {
        v[m] = gload_nt(src + (size_t)step * m, off);
        if (a.pre) v[m] = cmul(v[m], gload(a.pre, j));
      }
    }
  } else if (!HOOK) {
    // unconditional (every launched group is whole: batch*n1 is a multiple
    // of C), so the waits for the small loads above stay partial
    const float2* src = a.in + base;
    static_for<0, E>([&](auto ic) {
      constexpr int m = load_slot<N2, E>(decltype(ic)::value);
      v[m] = gload_nt(src + (size_t)step * m, off);
    });
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = make_float2(0.f, 0.f);
  }
  __builtin_amdgcn_sched_barrier(0);
  // LDS writes of the small tables; stage 0's exchange barriers order them
  // before their reads (stage 1's twiddles, the factor table in the store)
#pragma unroll
  for (int i = 0; i < FQ; ++i) {
    const int q = tid + NT * i;
    if ((C * E) % NT == 0 || q < C * E) ftab[(q / E) * FP + q % E] = cmul(fh[i], fl[i]);
  }
  if constexpr (LTW && !PERSIST) fs_store_tw1<N2, E, NT, TQ>(twl, tq, tid);
  if (valid && !HOOK && a.shift && (c1 & 1)) {  // element index c1 + n1*k has the parity of c1 (n1 even)
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = negate_bits(v[m]);
  }
  if constexpr (LTW) {
    const TwLdsStage<1> tws{a.tw, twl, (uint32_t)sched_tw_off(N2, E, 1)};
    run_stages<N2, E, S, false, L, SPLIT>(v, lds, tws, u, line);
  } else {
    run_stages<N2, E, S, false, L, SPLIT>(v, lds, a.tw, u, line);
  }
  if (valid) {
    // line, u and c1 again from an opaque copy of the thread index: kept live
    // across the stages they cost VGPRs (spills)
    int tid2 = tid;
    asm volatile("" : "+v"(tid2));
    const int line2 = tid2 % C, u2 = tid2 / C;
    const uint32_t eu = (c0 + (uint32_t)line2) * (uint32_t)u2;
    const float2 wu = cmul(gload(a.thi, eu >> a.bits), gload(a.tlo, eu & mask));
    // the block layout, relative to the first block column of this group.
    // Ordinary (not streaming) stores: pass 2 finds part of the scratch still
    // in the caches (2^22 x 32: 906 -> 891 us per exec; streaming loads or
    // ordinary stores in pass 2 were slower, 945 and 952 us)
    float2* dst = a.out + b * (int64_t)n1 * N2 + c0 * BK;
    if constexpr (T % BK == 0) {
      // k2 = u2 + T*m with T a multiple of BK: the block index is a
      // per-thread base plus m*T*n1 (whole block rows), a uniform stride
      const uint32_t base = fs_block_index<BK, C>((uint32_t)u2, (uint32_t)line2, n1);
      const size_t row_step = (size_t)T * n1;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        const float2 w = cmul(wu, ftab[line2 * FP + m]);
        gstore(dst + row_step * m, base, apply_tw<S>(v[m], w));
        if constexpr (E > 16) {
          if ((m & 7) == 7) __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < E; ++m) {
        const uint32_t k2 = (uint32_t)(u2 + T * m);
        const float2 w = cmul(wu, ftab[line2 * FP + m]);
        gstore(dst, fs_block_index<BK, C>(k2, (uint32_t)line2, n1), apply_tw<S>(v[m], w));
        if constexpr (E > 16) {
          if ((m & 7) == 7) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
  if constexpr (!PERSIST) break;  // one tile per workgroup
  lds_barrier();  // the next tile's factor table and exchanges overwrite LDS
  }
}

// ---------------------------------------------------------------------------
// Four-step pass 2: row transforms of length N1 over rows k2 of the block
// layout (BC: columns per pass-1 workgroup), element k1 stored at
// k2 + n2*k1.  The results go through LDS once more and come back out with
// consecutive threads on consecutive rows, so each store is a run of C
// elements.
//
// Tiles of 64 values per thread (N1 >= 2048: 8 waves hold the CU alone) are
// persistent: the grid holds as many workgroups as the CUs run at once, and
// each loops over tiles gridDim.x apart (in the XCD-grouped order).  A tile's
// strided stores then drain while the same workgroup issues the next tile's
// contiguous loads, instead of the CU waiting for a new workgroup, and the
// stage-1 twiddles are copied to LDS once per workgroup.  Measured per exec
// (512 MiB): 2^22 x 32 pass 2 459 -> 418 us, 2^22 x 16 493 -> 477 us, 2^24 x 4
// 764 -> 745 us, 2^28 14.63 -> 14.08 ms; the same loop in pass 1 no change.
// The smaller tiles (2^15 .. 2^20: 0.85x .. 0.99x when persistent) launch one
// workgroup per tile and run the loop once.  A staggered start as in pass 1
// made this pass slower (428 -> 428-441 us for 6-18 us).
// ---------------------------------------------------------------------------
template <int N1>
constexpr bool fs_rows_persistent() {
  return tile_e(N1, true) == kSplitValues;
}
template <int N1, int S, int BC>
__global__ __launch_bounds__(tile_lines(N1, true) * (N1 / tile_e(N1, true)))
__attribute__((amdgpu_waves_per_eu(fs_waves(N1)))) void k_fs_rows(FourStepArgs a) {
  constexpr int E = tile_e(N1, true);
  constexpr bool SPLIT = tile_split(N1, true);
  constexpr int C = tile_lines(N1, true);
  constexpr int T = N1 / E;
  constexpr int NT = C * T;
  constexpr bool WL = T <= 64;
  using L = RowLds<N1, SPLIT, E, true>;  // transposed read-back
  static_assert(L::size(C) * sizeof(lds_elem_t<SPLIT>) <= kLdsBudgetBytes, "LDS budget");
  constexpr int TW1 = fs_tw1_elems<N1, E>();
  constexpr bool LTW = sched_stages(N1, E) >= 2 &&
                       L::size(C) * sizeof(lds_elem_t<SPLIT>) + TW1 * sizeof(float2) <= kLdsBudgetBytes;
  __shared__ lds_elem_t<SPLIT> lds[L::size(C)];
  __shared__ float2 twl[LTW ? TW1 : 1];
  lds_poison(lds, twl);

  constexpr bool PERSIST = fs_rows_persistent<N1>();
  // stage-1 twiddles: copied to LDS once per workgroup when persistent; else
  // fetched before the line's loads and stored to LDS after them (see
  // k_fs_cols)
  constexpr int TQ = LTW ? (TW1 + NT - 1) / NT : 1;
  if constexpr (LTW && PERSIST) {
    float2 tq[TQ];
    fs_fetch_tw1<N1, E, NT, TQ>(tq, a.tw, threadIdx.x);
    fs_store_tw1<N1, E, NT, TQ>(twl, tq, threadIdx.x);
    lds_barrier();  // the stage exchanges may be wave-local: publish the copy here
  }
  const int64_t n2 = a.n2;
  const int64_t lines = a.batch * n2;
  const uint32_t ntiles = (uint32_t)(lines / C);  // whole groups (checked by the launcher)
  for (uint32_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
  // a per-tile opaque copy of the thread index: what derives from it is
  // recomputed per tile rather than kept live across the loop (spills)
  int tid = threadIdx.x;
  if constexpr (PERSIST) asm volatile("" : "+v"(tid));
  const int line = tid / T, u = tid % T;
  float2 tq[TQ];
  if constexpr (LTW && !PERSIST) fs_fetch_tw1<N1, E, NT, TQ>(tq, a.tw, tid);
  __builtin_amdgcn_sched_barrier(0);
  const int64_t g0 = (int64_t)xcd_grouped_block(tile, ntiles) * C;
  float2 v[E];
  {
    // rows k2 = k20 .. k20 + C - 1 of transform b form one row of blocks
    // starting at (b*n2 + k20)*N1 (k20 is a multiple of C).  Unconditional:
    // every launched group is whole (batch*n2 is a multiple of C).
    const float2* src = a.in + g0 * N1;
    if constexpr (T % BC == 0) {
      // slot m adds T/BC whole blocks: a compile-time step of the base
      const uint32_t off = fs_block_index<C, BC>((uint32_t)line, (uint32_t)u, N1);
      static_for<0, E>([&](auto ic) {
        constexpr int m = load_slot<N1, E>(decltype(ic)::value);
        v[m] = gload_nt(src + (T / BC) * C * BC * m, off);
      });
    } else {
      static_for<0, E>([&](auto ic) {
        constexpr int m = load_slot<N1, E>(decltype(ic)::value);
        v[m] = gload_nt(src, fs_block_index<C, BC>((uint32_t)line, (uint32_t)(u + T * m), N1));
      });
    }
  }
  if constexpr (LTW) {
    if constexpr (!PERSIST) {
      __builtin_amdgcn_sched_barrier(0);
      fs_store_tw1<N1, E, NT, TQ>(twl, tq, tid);
      lds_barrier();  // the stage exchanges may be wave-local: publish the copy here
    }
    const TwLdsStage<1> tws{a.tw, twl, (uint32_t)sched_tw_off(N1, E, 1)};
    run_stages<N1, E, S, WL, L, SPLIT>(v, lds, tws, u, line);
  } else {
    run_stages<N1, E, S, WL, L, SPLIT>(v, lds, a.tw, u, line);
  }
  // transposed read-back: slot p of thread tid is q = tid + NT*p, i.e. line
  // q % C = tid % C and element q / C = tid / C + (NT / C) * p (NT is a
  // multiple of C)
  lds_barrier();
  static_assert(NT % C == 0, "transposed read-back layout");
  if constexpr (SPLIT) {
    static_for<0, E>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      lds[L::template at_k<T * m>(line, u)] = v[m].x;
    });
    lds_barrier();
    static_for<0, E>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      v[p].x = lds[L::template at_k<(NT / C) * p>(tid % C, tid / C)];
    });
    lds_barrier();
    int u2 = u, line2 = line, tid2 = tid;  // recompute addresses (see run_stage)
    asm volatile("" : "+v"(u2), "+v"(line2), "+v"(tid2));
    static_for<0, E>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      lds[L::template at_k<T * m>(line2, u2)] = v[m].y;
    });
    lds_barrier();
    static_for<0, E>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      v[p].y = lds[L::template at_k<(NT / C) * p>(tid2 % C, tid2 / C)];
    });
  } else {
    static_for<0, E>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      lds[L::template at_k<T * m>(line, u)] = v[m];
    });
    lds_barrier();
    static_for<0, E>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      v[p] = lds[L::template at_k<(NT / C) * p>(tid % C, tid / C)];
    });
  }
  const int ln = tid % C;  // the same line for every slot p (NT is a multiple of C)
  if (g0 + ln < lines) {
    // n2 >= 128 > C: the group's rows belong to one transform b.  n2 is a
    // power of two: shifts, not a 64-bit division (whose reciprocal the
    // compiler would keep live across the tile loop)
    const uint32_t n2_log2 = (uint32_t)__builtin_ctzll((uint64_t)n2);
    const int64_t b = g0 >> n2_log2;
    const int64_t k20 = g0 & (n2 - 1);
    float2* dst = a.out + b * n2 * N1 + k20;
    const uint32_t off = (uint32_t)ln + (uint32_t)(tid / C) * (uint32_t)n2;
    const size_t step = (size_t)(NT / C) * (size_t)n2;
#pragma unroll
    for (int p = 0; p < E; ++p) {
      gstore_nt(dst + step * p, off, v[p]);
      if constexpr (E > 16) {
        if ((p & 7) == 7) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (!PERSIST) break;  // one tile per workgroup
  lds_barrier();  // the next tile's exchanges overwrite LDS
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

// Workgroups of KERNEL (launched with `threads` threads and no dynamic LDS)
// that the current device runs at once: CUs x resident workgroups per CU,
// queried once per device.  Grid size of the persistent kernels.
constexpr int kResidentDevices = 64;
template <auto KERNEL>
hipError_t resident_workgroups(int threads, uint32_t* out) {
  static std::atomic<uint32_t> cache[kResidentDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cacheable = dev >= 0 && dev < kResidentDevices;
  if (cacheable) {
    const uint32_t c = cache[dev].load(std::memory_order_relaxed);
    if (c) {
      *out = c;
      return hipSuccess;
    }
  }
  int per_cu = 0, cus = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KERNEL, threads, 0)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if (per_cu < 1 || cus < 1) return hipErrorInvalidConfiguration;
  const uint32_t r = (uint32_t)per_cu * (uint32_t)cus;
  if (cacheable) cache[dev].store(r, std::memory_order_relaxed);
  *out = r;
  return hipSuccess;
}

// The stagger of a persistent launch: `us` microseconds in wall-clock ticks
// of the current device, when each workgroup runs at least 4 tiles (else 0:
// a delayed workgroup would only lengthen the launch).
inline hipError_t stagger_ticks(double us, uint32_t tiles, uint32_t grid, int64_t* out) {
  static std::atomic<int> rate_khz[kResidentDevices];
  *out = 0;
  if ((uint64_t)tiles < 4ull * grid) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int khz = dev >= 0 && dev < kResidentDevices ? rate_khz[dev].load(std::memory_order_relaxed) : 0;
  if (khz == 0) {
    if ((e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess) return e;
    if (khz <= 0) return hipSuccess;  // no wall clock: no stagger
    if (dev >= 0 && dev < kResidentDevices) rate_khz[dev].store(khz, std::memory_order_relaxed);
  }
  *out = (int64_t)(us * khz / 1000.0);
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
