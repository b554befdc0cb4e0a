// stockham.hpp -- device building blocks of the natural-order Stockham FFT for
// gfx950 (CDNA4, wave64).
//
// One transform line (a row, a column, or a four-step sub-transform) of length
// N is held by T = N/E threads, E complex values each, in registers.  Thread u
// always owns elements u + T*m, m = 0..E-1 ("slot m"), at the start and at the
// end of every stage, so the first stage reads straight from HBM and the last
// stage writes straight to HBM, both coalesced.  Between stages the values go
// through LDS once (write, barrier, read, barrier).
//
// Stage s has radix R (16, or the leftover 2/4/8 as the last stage) and
// NS = product of the radices before it.  Butterfly b reads elements
// b + r*N/R, multiplies element r by W^{r*j} with W = e^{sign 2 pi i/(NS*R)}
// and j = b mod NS, runs an R-point DFT and writes output q to
// (b - j)*R + j + q*NS.  This is the radix-R form of the autosort stages in
// the WGSL Fourier-stage source (turing-sphere fourier.ts, stockham() and
// stockham4()) and of the radix-4 Stockham dragonfly of "High Performance
// Fourier Transforms on GPUs with GLSL" (Mota, section 2.5, Equation 15).
// Twiddles come from a table built on the host in f64 and rounded once to
// fp32 (fourier.ts header: device sin/cos would dominate the fp32 error).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fftamd {

// ---------------------------------------------------------------------------
// schedule (shared by host table construction and device templates)
// ---------------------------------------------------------------------------
constexpr int ilog2c(int64_t n) {
  int l = 0;
  while ((int64_t(1) << l) < n) ++l;
  return l;
}
// values held per thread
constexpr int sched_e(int n) { return n < 16 ? n : 16; }
// number of radix-16 stages and the leftover radix (1 = none)
constexpr int sched_n16(int n) { return n < 16 ? 0 : ilog2c(n) / 4; }
constexpr int sched_rem(int n) { return n < 16 ? n : (1 << (ilog2c(n) % 4)); }
constexpr int sched_stages(int n) { return sched_n16(n) + (sched_rem(n) > 1 ? 1 : 0); }
constexpr int sched_radix(int n, int s) { return s < sched_n16(n) ? 16 : sched_rem(n); }
constexpr int sched_ns(int n, int s) {
  int p = 1;
  for (int t = 0; t < s; ++t) p *= sched_radix(n, t);
  return p;
}
// offset of stage s in the twiddle table (stage 0 needs none)
constexpr int sched_tw_off(int n, int s) {
  int o = 0;
  for (int t = 1; t < s; ++t) o += (sched_radix(n, t) - 1) * sched_ns(n, t);
  return o;
}
constexpr int sched_tw_size(int n) { return sched_tw_off(n, sched_stages(n)); }

// Longest line held in one workgroup: 16384 complex = 128 KiB (+1/16 padding)
// of the 160 KiB of LDS a gfx950 workgroup may use.
constexpr int kMaxSinglePass = 16384;
constexpr int kMaxThreads = 1024;
constexpr int kLdsBudgetBytes = 160 * 1024;

// ---------------------------------------------------------------------------
// complex arithmetic
// ---------------------------------------------------------------------------
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
// a * conj(b)
__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {
  return make_float2(a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y);
}
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
// multiply by S*i
template <int S>
__device__ __forceinline__ float2 mul_si(float2 v) {
  return S > 0 ? make_float2(-v.y, v.x) : make_float2(v.y, -v.x);
}
// twiddle from a forward table entry (e^{-...}): itself for the forward
// transform, its conjugate for the inverse
template <int S>
__device__ __forceinline__ float2 apply_tw(float2 v, float2 w) {
  return S < 0 ? cmul(v, w) : cmulc(v, w);
}

// flip the sign bits of both parts: exact multiplication by -1
__device__ __forceinline__ float2 negate_bits(float2 v) {
  return make_float2(__uint_as_float(__float_as_uint(v.x) ^ 0x80000000u),
                     __uint_as_float(__float_as_uint(v.y) ^ 0x80000000u));
}

// ---------------------------------------------------------------------------
// constant twiddles of the in-register DFTs (R <= 16), in units of 2*pi/16
// cos(pi/4), cos(pi/8), sin(pi/8) written to 20 digits, rounded once to fp32
// ---------------------------------------------------------------------------
#define FFTAMD_C8 0.70710678118654752440f
#define FFTAMD_C16 0.92387953251128675613f
#define FFTAMD_S16 0.38268343236508977173f

__host__ __device__ constexpr float cos16(int k) {
  switch (k & 15) {
    case 0: return 1.0f;
    case 1: return FFTAMD_C16;
    case 2: return FFTAMD_C8;
    case 3: return FFTAMD_S16;
    case 4: return 0.0f;
    case 5: return -FFTAMD_S16;
    case 6: return -FFTAMD_C8;
    case 7: return -FFTAMD_C16;
    case 8: return -1.0f;
    case 9: return -FFTAMD_C16;
    case 10: return -FFTAMD_C8;
    case 11: return -FFTAMD_S16;
    case 12: return 0.0f;
    case 13: return FFTAMD_S16;
    case 14: return FFTAMD_C8;
    default: return FFTAMD_C16;
  }
}
__host__ __device__ constexpr float sin16(int k) { return cos16(k - 4); }

// v * e^{S * 2*pi*i * K/R}, K and R compile-time, R | 16
template <int R, int K, int S>
__device__ __forceinline__ float2 twc(float2 v) {
  constexpr int k = ((K * (16 / R)) % 16 + 16) % 16;
  if constexpr (k == 0) {
    return v;
  } else if constexpr (k == 4) {
    return mul_si<S>(v);
  } else if constexpr (k == 8) {
    return make_float2(-v.x, -v.y);
  } else if constexpr (k == 12) {
    return mul_si<-S>(v);
  } else if constexpr ((k & 1) == 0) {
    // odd multiple of pi/4: both parts of the factor have magnitude cos(pi/4)
    constexpr float sc = cos16(k) > 0 ? 1.0f : -1.0f;
    constexpr float ss = (S > 0 ? 1.0f : -1.0f) * (sin16(k) > 0 ? 1.0f : -1.0f);
    return make_float2(FFTAMD_C8 * (sc * v.x - ss * v.y), FFTAMD_C8 * (ss * v.x + sc * v.y));
  } else {
    constexpr float c = cos16(k);
    constexpr float s = (S > 0 ? 1.0f : -1.0f) * sin16(k);
    return make_float2(v.x * c - v.y * s, v.x * s + v.y * c);
  }
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// In-register R-point DFT, natural order in and out:
// y_k = sum_j x_j e^{S 2 pi i jk/R}.  R = 2 and 4 are written out (Mota,
// section 2.3, Equations 7-8); 8 and 16 split into even and odd halves
// (section 2.3.1, Equation 9).
template <int R, int S>
__device__ __forceinline__ void dft(float2* x) {
  if constexpr (R == 1) {
  } else if constexpr (R == 2) {
    float2 a = x[0], b = x[1];
    x[0] = cadd(a, b);
    x[1] = csub(a, b);
  } else if constexpr (R == 4) {
    float2 a = cadd(x[0], x[2]);
    float2 b = csub(x[0], x[2]);
    float2 c = cadd(x[1], x[3]);
    float2 d = mul_si<S>(csub(x[1], x[3]));
    x[0] = cadd(a, c);
    x[1] = cadd(b, d);
    x[2] = csub(a, c);
    x[3] = csub(b, d);
  } else {
    constexpr int H = R / 2;
    float2 e[H], o[H];
#pragma unroll
    for (int i = 0; i < H; ++i) {
      e[i] = x[2 * i];
      o[i] = x[2 * i + 1];
    }
    dft<H, S>(e);
    dft<H, S>(o);
    static_for<0, H>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      float2 t = twc<R, k, S>(o[k]);
      x[k] = cadd(e[k], t);
      x[k + H] = csub(e[k], t);
    });
  }
}

// ---------------------------------------------------------------------------
// LDS addressing.  Lines of one workgroup are stored either one after the
// other (row lanes: consecutive threads walk along a line) or interleaved
// (column lanes: consecutive threads walk across lines).  One float2 of
// padding every 16 breaks the power-of-two strides of the Stockham writes
// over the LDS banks; row-lane lines are also offset by one element from each
// other so that reading across lines (transposing stores) does not collide.
// ---------------------------------------------------------------------------
template <int N>
struct RowLds {
  static constexpr int kStride = N + (N >> 4) + 1;
  __device__ __forceinline__ static int at(int line, int i) { return line * kStride + i + (i >> 4); }
  static constexpr int size(int lines) { return lines * kStride; }
};
template <int N, int C>
struct ColLds {
  __device__ __forceinline__ static int at(int line, int i) {
    int a = i * C + line;
    return a + (a >> 4);
  }
  static constexpr int size(int lines) { return N * C + ((N * C) >> 4) + 1; }
};

// Barrier between the LDS writes and reads of one exchange.  When every line
// of the workgroup sits inside one wavefront, a wave-level barrier suffices.
template <bool WAVE_LOCAL>
__device__ __forceinline__ void lds_sync() {
  if constexpr (WAVE_LOCAL) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  } else {
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// the stages.  On entry and exit v[m] holds element u + T*m of `line`.
// tw: forward twiddles of all stages (stage s, factor r, index j at
// sched_tw_off(N,s) + (r-1)*NS + j holds e^{-2 pi i r j/(NS*R)}).
// On return other threads may still be reading LDS: synchronise before
// writing it again.
// ---------------------------------------------------------------------------
template <int N, int S, bool WAVE_LOCAL, class Lds>
__device__ __forceinline__ void run_stages(float2* v, float2* lds, const float2* __restrict__ tw,
                                           int u, int line) {
  constexpr int E = sched_e(N);
  constexpr int T = N / E;
  constexpr int NST = sched_stages(N);
  static_for<0, NST>([&](auto sc) {
    constexpr int s = decltype(sc)::value;
    constexpr int R = sched_radix(N, s);
    constexpr int NS = sched_ns(N, s);
    constexpr int KB = E / R;
    constexpr bool last = (s == NST - 1);
    constexpr int OFF = sched_tw_off(N, s);
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      float2 x[R];
#pragma unroll
      for (int r = 0; r < R; ++r) x[r] = v[k + r * KB];
      const int b = u + T * k;
      const int j = b & (NS - 1);
      if constexpr (s > 0) {
#pragma unroll
        for (int r = 1; r < R; ++r) x[r] = apply_tw<S>(x[r], tw[OFF + (r - 1) * NS + j]);
      }
      dft<R, S>(x);
      if constexpr (last) {
#pragma unroll
        for (int r = 0; r < R; ++r) v[k + r * KB] = x[r];
      } else {
        const int base = (b - j) * R + j;
#pragma unroll
        for (int r = 0; r < R; ++r) lds[Lds::at(line, base + r * NS)] = x[r];
      }
    }
    if constexpr (!last) {
      lds_sync<WAVE_LOCAL>();
#pragma unroll
      for (int m = 0; m < E; ++m) v[m] = lds[Lds::at(line, u + T * m)];
      if constexpr (s + 1 < NST - 1) lds_sync<WAVE_LOCAL>();
    }
  });
}

}  // namespace fftamd
