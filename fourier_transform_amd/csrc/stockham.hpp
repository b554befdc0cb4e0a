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
// Default values held per thread (row kernels): 16.
constexpr int sched_e(int n) { return n < 16 ? n : 16; }
// Radix schedule for E values per thread.  The first stage (no twiddles)
// takes radix min(E, 64, n); later stages take radix min(E, 32) and the
// leftover power of two comes last.  With E = 16 this is all radix 16; with
// E = 64 a 2048-point line is 64 x 32, one LDS exchange.  A twiddled radix-64
// stage would need more than 256 VGPRs, hence the cap of 32 after stage 0.
constexpr int sched_r0(int n, int e) {
  int r = e < 64 ? e : 64;
  return r < n ? r : n;
}
constexpr int sched_rmax(int e) { return e < 32 ? e : 32; }
constexpr int sched_nfull(int n, int e) {
  return ilog2c(n / sched_r0(n, e)) / ilog2c(sched_rmax(e));
}
constexpr int sched_rem(int n, int e) {
  return 1 << (ilog2c(n / sched_r0(n, e)) % ilog2c(sched_rmax(e)));
}
constexpr int sched_stages(int n, int e) { return 1 + sched_nfull(n, e) + (sched_rem(n, e) > 1 ? 1 : 0); }
constexpr int sched_radix(int n, int e, int s) {
  return s == 0 ? sched_r0(n, e) : (s - 1 < sched_nfull(n, e) ? sched_rmax(e) : sched_rem(n, e));
}
constexpr int sched_ns(int n, int e, int s) {
  int p = 1;
  for (int t = 0; t < s; ++t) p *= sched_radix(n, e, t);
  return p;
}
// offset of stage s in the twiddle table (stage 0 needs none)
constexpr int sched_tw_off(int n, int e, int s) {
  int o = 0;
  for (int t = 1; t < s; ++t) o += (sched_radix(n, e, t) - 1) * sched_ns(n, e, t);
  return o;
}
constexpr int sched_tw_size(int n, int e) { return sched_tw_off(n, e, sched_stages(n, e)); }

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

// Global accesses as a wave-uniform base pointer plus an unsigned 32-bit
// element offset: the compiler then uses the SGPR-base form of the global
// memory instructions (one 32-bit VGPR per address instead of a 64-bit pair
// built with 64-bit multiply-adds).  Offsets must stay below 2^29 elements.
// Where an unrolled loop steps by a compile-time or wave-uniform stride, the
// callers add the stride to the base pointer (scalar arithmetic) and keep one
// per-thread offset for every access: the instruction's immediate offset
// only reaches 4 KiB, so folding the stride into the offset costs one or
// two vector adds per access.
__device__ __forceinline__ float2 gload(const float2* __restrict__ base, uint32_t i) {
  return *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(base) + (i << 3));
}
__device__ __forceinline__ void gstore(float2* base, uint32_t i, float2 v) {
  *reinterpret_cast<float2*>(reinterpret_cast<char*>(base) + (i << 3)) = v;
}
// Streaming variants (non-temporal hint) for data touched once.  Used where
// measurement shows they help: loads of whole rows and of column-stage
// segments, stores of whole rows, and both directions of the four-step
// passes.  Not for the 2D column pass, whose 32 B runs rely on neighbouring
// workgroups meeting in L2.
typedef float fftamd_v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float2 gload_nt(const float2* __restrict__ base, uint32_t i) {
  const fftamd_v2f w = __builtin_nontemporal_load(
      reinterpret_cast<const fftamd_v2f*>(reinterpret_cast<const char*>(base) + (i << 3)));
  return make_float2(w.x, w.y);
}
__device__ __forceinline__ void gstore_nt(float2* base, uint32_t i, float2 v) {
  const fftamd_v2f w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<fftamd_v2f*>(reinterpret_cast<char*>(base) + (i << 3)));
}

// flip the sign bits of both parts: exact multiplication by -1
__device__ __forceinline__ float2 negate_bits(float2 v) {
  return make_float2(__uint_as_float(__float_as_uint(v.x) ^ 0x80000000u),
                     __uint_as_float(__float_as_uint(v.y) ^ 0x80000000u));
}

// ---------------------------------------------------------------------------
// constant twiddles of the in-register DFTs (R <= 64), in units of 2*pi/64:
// cos(pi*k/32), k = 0..16, written to 22 digits and rounded once to fp32
// ---------------------------------------------------------------------------
__host__ __device__ constexpr float cos64_q(int k) {  // 0 <= k <= 16
  switch (k) {
    case 0: return 1.0f;
    case 1: return 0.9951847266721968862448f;
    case 2: return 0.9807852804032304491262f;
    case 3: return 0.9569403357322088649358f;
    case 4: return 0.9238795325112867561282f;
    case 5: return 0.8819212643483550297128f;
    case 6: return 0.8314696123025452370788f;
    case 7: return 0.7730104533627369608109f;
    case 8: return 0.7071067811865475244008f;
    case 9: return 0.6343932841636454982152f;
    case 10: return 0.5555702330196022247428f;
    case 11: return 0.4713967368259976485564f;
    case 12: return 0.3826834323650897717285f;
    case 13: return 0.2902846772544623676362f;
    case 14: return 0.1950903220161282678483f;
    case 15: return 0.0980171403295606019942f;
    default: return 0.0f;
  }
}
// cos(2*pi*k/64) for any k, by the symmetries of the quarter wave
__host__ __device__ constexpr float cos64(int k) {
  k &= 63;
  if (k <= 16) return cos64_q(k);
  if (k <= 32) return -cos64_q(32 - k);
  if (k <= 48) return -cos64_q(k - 32);
  return cos64_q(64 - k);
}
__host__ __device__ constexpr float sin64(int k) { return cos64(k - 16); }

// v * e^{S * 2*pi*i * K/R}, K and R compile-time, R | 64
template <int R, int K, int S>
__device__ __forceinline__ float2 twc(float2 v) {
  constexpr int k = ((K * (64 / R)) % 64 + 64) % 64;
  if constexpr (k == 0) {
    return v;
  } else if constexpr (k == 16) {
    return mul_si<S>(v);
  } else if constexpr (k == 32) {
    return make_float2(-v.x, -v.y);
  } else if constexpr (k == 48) {
    return mul_si<-S>(v);
  } else if constexpr ((k & 15) == 8) {
    // odd multiple of pi/4: both parts of the factor have magnitude cos(pi/4)
    constexpr float c8 = cos64_q(8);
    constexpr float sc = cos64(k) > 0 ? 1.0f : -1.0f;
    constexpr float ss = (S > 0 ? 1.0f : -1.0f) * (sin64(k) > 0 ? 1.0f : -1.0f);
    return make_float2(c8 * (sc * v.x - ss * v.y), c8 * (ss * v.x + sc * v.y));
  } else {
    constexpr float c = cos64(k);
    constexpr float s = (S > 0 ? 1.0f : -1.0f) * sin64(k);
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
// (section 2.3.1, Equation 9); 32 = 4 x 8 and 64 = 8 x 8 use the same
// two-factor split as the four-step pass (transforms over the coarse index,
// constant twiddles, transforms over the fine index), all indices compile-time.
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
  } else if constexpr (R <= 16) {
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
  } else {
    // R = A*B, input index a + A*b, output index kb + B*ka
    constexpr int A = R == 32 ? 4 : 8;
    constexpr int B = R / A;
    float2 y[R];
    static_for<0, A>([&](auto ac) {
      constexpr int a = decltype(ac)::value;
      float2 t[B];
#pragma unroll
      for (int b = 0; b < B; ++b) t[b] = x[a + A * b];
      dft<B, S>(t);
      static_for<0, B>([&](auto kc) {
        constexpr int kb = decltype(kc)::value;
        y[a + A * kb] = twc<R, a * kb, S>(t[kb]);
      });
    });
    static_for<0, B>([&](auto kc) {
      constexpr int kb = decltype(kc)::value;
      float2 t[A];
#pragma unroll
      for (int a = 0; a < A; ++a) t[a] = y[a + A * kb];
      dft<A, S>(t);
#pragma unroll
      for (int ka = 0; ka < A; ++ka) x[kb + B * ka] = t[ka];
    });
  }
}

// ---------------------------------------------------------------------------
// LDS addressing.  Lines of one workgroup are stored either one after the
// other (row lanes: consecutive threads walk along a line) or interleaved
// (column lanes: consecutive threads walk across lines).  Indices are padded
// so that the power-of-two strides of the Stockham writes, the slot reads and
// the transposed reads spread over the banks.  The bank model for reads and
// 4-byte accesses, fitted to the SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE
// counters of these kernels and of probes with fixed access patterns on
// gfx950: a clock's cost is the largest number of distinct dwords on one
// bank; 8-byte reads serve 32 lanes per clock over 64 banks, 4-byte accesses
// 32 lanes per clock over 32 banks.  (The 8-byte writes of the first stage,
// lanes 16 elements apart, still cost one extra clock in four whichever
// padding period of 16, 32 or 64 is used; that was measured, not modelled.)
//   row lanes:            line * P + p(i),  p(i) = i + i/G.
//                         8-byte: G = 32, so 32 consecutive elements stay in
//                         one block of the 64 banks.  P = T mod 32 for lines
//                         of 1 < T < 32 threads, so the lines that share a
//                         clock tile the banks; lines of one thread exchange
//                         nothing and take P = p(N) + 1 (real rows of 32:
//                         per 1 GiB of reals R2C 508 -> 420 us, C2R 618 ->
//                         495, from the LDS no longer limiting occupancy).  Lines that are also read across
//                         (the transposed read-back of the four-step row
//                         pass: 16 lines at two neighbouring indices per
//                         clock) take P = 6 mod 32, best for every T there.
//                         4-byte: G = E (32 or 64), the stride between the
//                         lanes of a first-stage write; P = 2 mod 32, so the
//                         16 lines of a read-back clock fill the 32 banks.
//   column lanes, 8-byte: p(a) = a + a/32 + 8*(a/256),  a = i*C + line
//   column lanes, 4-byte: p(a) = a + a/64
// SPLIT: the exchange moves 4-byte halves (real, then imaginary parts).
//
// at_k<K, A>(line, i0) addresses element i0 + K, where K is a compile-time
// constant (the r*NS and T*m offsets of the unrolled loops) and the runtime
// part i0 is a multiple of A.  Each padding is additive over multiples of its
// period M (p(x + M q) = p(x) + p(M q)), so only K mod M enters the runtime
// arithmetic -- and of that only the part above the alignment A -- and the
// rest becomes the immediate offset of the LDS instruction.  The unrolled
// loops then share a handful of runtime addresses instead of padding every
// index separately.
// ---------------------------------------------------------------------------
constexpr int row_pad_g(bool split, int e) { return split && e >= 64 ? 64 : 32; }
constexpr int row_pad(int i, bool split, int e) { return i + i / row_pad_g(split, e); }
// xread: lines are also read across (16 lines at two neighbouring indices)
constexpr int row_pitch(int n, bool split, int e, bool xread) {
  const int p = row_pad(n, split, e) + 1;
  const int t = n / e;
  if (t == 1) return p;  // lines of one thread: no exchange, the pitch only separates them
  const int target = split ? 2 : xread ? 6 : t < 32 ? t : 1;
  return p + ((target - p % 32) % 32 + 32) % 32;
}
constexpr int row_lds_elems(int n, int lines, bool split, int e, bool xread = false) {
  return (lines - 1) * row_pitch(n, split, e, xread) + row_pad(n - 1, split, e) + 1;
}
template <bool SPLIT>
__host__ __device__ constexpr uint32_t col_pad(uint32_t a) {
  return SPLIT ? a + a / 64 : a + a / 32 + 8 * (a / 256);
}
constexpr int col_lds_elems(int n, int lines, bool split) {
  return (int)(split ? col_pad<true>((uint32_t)(n * lines - 1)) : col_pad<false>((uint32_t)(n * lines - 1))) + 1;
}

template <int N, bool SPLIT = false, int E = 16, bool XREAD = false>
struct RowLds {
  static constexpr uint32_t G = row_pad_g(SPLIT, E);
  static constexpr uint32_t P = row_pitch(N, SPLIT, E, XREAD);
  __host__ __device__ static constexpr uint32_t pad(uint32_t i) { return i + i / G; }
  __device__ __forceinline__ static int at(int line, int i) {
    return (int)((uint32_t)line * P + pad((uint32_t)i));
  }
  template <int K, int A = 1>
  __device__ __forceinline__ static int at_k(int line, int i0) {
    constexpr uint32_t r = (uint32_t)K % G;      // part of K below the period
    constexpr uint32_t ra = r - r % (uint32_t)A;  // ... that can carry into i0's padding
    constexpr uint32_t q = (uint32_t)K - r;
    return (int)((uint32_t)line * P + pad((uint32_t)i0 + ra) + (r - ra) + pad(q));
  }
  static constexpr int size(int lines) { return row_lds_elems(N, lines, SPLIT, E, XREAD); }
};
template <int N, int C, bool SPLIT = false>
struct ColLds {
  static constexpr uint32_t M = SPLIT ? 64 : 256;
  __device__ __forceinline__ static int at(int line, int i) {
    return (int)col_pad<SPLIT>((uint32_t)i * C + (uint32_t)line);
  }
  template <int K, int A = 1>
  __device__ __forceinline__ static int at_k(int line, int i0) {
    constexpr uint32_t kc = (uint32_t)K * C;
    constexpr uint32_t r = kc % M;
    return (int)(col_pad<SPLIT>((uint32_t)i0 * C + (uint32_t)line + r) + col_pad<SPLIT>(kc - r));
  }
  static constexpr int size(int lines) { return col_lds_elems(N, C, SPLIT); }
};

// Runtime part and compile-time offset of the Stockham write address of
// butterfly k (element (b - j)*R + j + r*NS, b = u + T*k, j = b mod NS).
// When NS divides T, b - j = (u - u mod NS) + T*k and the runtime part is the
// same for every k; in the first stage (NS = 1) it is u*R, a multiple of R.
template <int T, int R, int NS, int k>
struct StageIdx {
  static constexpr bool kShared = T % NS == 0;
  static constexpr int K0 = kShared ? T * k * R : 0;
  static constexpr int A = (kShared && NS == 1) ? R : 1;
  __device__ __forceinline__ static int base(int u) {
    if constexpr (kShared) {
      const int jn = u & (NS - 1);
      return (u - jn) * R + jn;
    } else {
      const int b = u + T * k;
      const int j = b & (NS - 1);
      return (b - j) * R + j;
    }
  }
};

// LDS-poison debug build (compiled with -DFFTAMD_LDS_POISON=1, the library
// libfft_amd_poison.so): every kernel first fills its LDS arrays with quiet
// NaNs and synchronises, so that a read of LDS that no thread of the
// workgroup has written in this kernel -- a missing barrier, a wrong index, a
// read of a pad element -- turns the output into NaNs instead of reusing a
// stale value left by an earlier workgroup.  (The hazard: the radix-2 kernel
// of the "Fast Fourier Transform on CPU and GPU" page loads shared memory and
// stores back into it with no barrier in between.)  In the default build the
// calls compile to nothing.
#ifndef FFTAMD_LDS_POISON
#define FFTAMD_LDS_POISON 0
#endif
__device__ __forceinline__ void lds_poison_bytes(void* p, uint32_t bytes) {
  if constexpr (FFTAMD_LDS_POISON != 0) {
    uint32_t* w = static_cast<uint32_t*>(p);
    const uint32_t nt = blockDim.x * blockDim.y * blockDim.z;
    const uint32_t t = threadIdx.x + blockDim.x * (threadIdx.y + blockDim.y * threadIdx.z);
    for (uint32_t i = t; i < bytes / 4; i += nt) w[i] = 0x7fc00000u;
  }
}
// static __shared__ arrays (sizes from their types), then a workgroup barrier
template <class... A>
__device__ __forceinline__ void lds_poison(A&... arrays) {
  if constexpr (FFTAMD_LDS_POISON != 0) {
    (lds_poison_bytes(static_cast<void*>(&arrays), (uint32_t)sizeof(arrays)), ...);
    __syncthreads();
  }
}
// dynamic LDS of `bytes` bytes, then a workgroup barrier
__device__ __forceinline__ void lds_poison_dynamic(void* p, uint32_t bytes) {
  if constexpr (FFTAMD_LDS_POISON != 0) {
    lds_poison_bytes(p, bytes);
    __syncthreads();
  }
}

// Barrier between the LDS writes and reads of one exchange.  The fences are
// restricted to LDS ("local" address space), so the barrier waits for LDS
// traffic only and leaves global loads in flight (prefetching kernels rely on
// this).  When every line of the workgroup sits inside one wavefront, a
// wave-level barrier suffices.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
template <bool WAVE_LOCAL>
__device__ __forceinline__ void lds_sync() {
  if constexpr (WAVE_LOCAL) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  } else {
    lds_barrier();
  }
}

// Order in which a thread loads its E values of a line from HBM: the order
// in which the first stage consumes them.  Butterfly k of that stage reads
// slots k + r*KB; dft() takes R = 32 and 64 as R = A*B and transforms the
// inputs a + A*b for one a at a time, and R = 8 and 16 as the even half, then
// the odd half.  Loads return in issue order, so the first sub-transform can
// start while the later loads are still in flight.
constexpr int dft_use_order(int R, int i) {
  if (R == 32 || R == 64) {
    const int A = R == 32 ? 4 : 8, B = R / A;
    return i / B + A * (i % B);
  }
  if (R == 8 || R == 16) return 2 * (i % (R / 2)) + i / (R / 2);
  return i;
}
template <int N, int E>
constexpr int load_slot(int i) {
  constexpr int R = sched_r0(N, E), KB = E / R;
  return i / R + KB * dft_use_order(R, i % R);
}

// ---------------------------------------------------------------------------
// the stages.  E values per thread (E a multiple of every radix, T = N/E
// threads per line).  On entry and exit v[m] holds element u + T*m of `line`.
// tw: forward twiddles of all stages (stage s, factor r, index j at
// sched_tw_off(N,s) + (r-1)*NS + j holds e^{-2 pi i r j/(NS*R)}).
// SPLIT = false: LDS holds float2 and one exchange is write, barrier, read.
// SPLIT = true: LDS holds floats and the real parts are exchanged, then the
// imaginary parts, so a workgroup can hold twice as many lines in the same
// LDS; the butterfly outputs wait in v meanwhile, so no extra registers.
// On return other threads may still be reading LDS: synchronise before
// writing it again.
// ---------------------------------------------------------------------------
// Twiddle sources of the stages: the table in global memory (a plain
// pointer), or TwLdsStage<LS>, which reads stage LS from a copy of that
// stage's part of the table in LDS (the copy starts at table offset `off`)
// and the other stages from global memory.
template <int LS>
struct TwLdsStage {
  const float2* __restrict__ g;
  const float2* l;
  uint32_t off;
};
// entry k + j of the table: k compile-time (folded into the base pointer),
// j per thread
template <int s>
__device__ __forceinline__ float2 tw_at(const float2* __restrict__ t, uint32_t k, uint32_t j) {
  return gload(t + k, j);
}
template <int s, int LS>
__device__ __forceinline__ float2 tw_at(const TwLdsStage<LS>& t, uint32_t k, uint32_t j) {
  if constexpr (s == LS) {
    return t.l[k - t.off + j];
  } else {
    return gload(t.g + k, j);
  }
}

// Exchanges inside a wavefront without LDS (gfx950 v_permlane32_swap and
// v_permlane16_swap).  After a radix-16 stage with NS = 16 and one 16-value
// butterfly per thread on a line of T = 64 (or 32) threads, thread
// u = 16c + j holds outputs q of element 256c + 16q + j.  The next stage wants
// element e on lane e mod T, slot e / T: lane 16(q mod 4) + j, slot 4c + q/4
// for T = 64 (lane 16(q mod 2) + j, slot 8c + q/2 for T = 32).  So the
// exchange only swaps the lane bits above 3 (c) with the low register bits
// (q mod 4, or q mod 2) and relabels the registers: permlane32_swap swaps
// lanes 32-63 of one register with lanes 0-31 of another (lane bit 5),
// permlane16_swap the odd 16-lane rows of one with the even rows of another
// (lane bit 4).  Lines of 32 threads are half-waves, so each swap stays
// inside its line.  Two (or one) rounds of 16 swaps replace 32 LDS accesses,
// their address arithmetic and a barrier.  Measured on MI355X against the
// LDS exchange: LDS instructions -58 % (1024-point rows) and -25 % (1024-point
// real transforms), VALU instructions +1.5 %, time equal or lower (1024 x 8:
// 4.2 against 4.5-5.1 us; real 2048 x 1024: 9.97 against 10.15 us per exec).
// The first exchange of these lines (NS = 1) also rotates the lane bits, so
// it stays in LDS: as swaps it would need six or more rounds, four of them at
// lane distances below 16 (DPP moves and selects, two to three instructions
// per value) or cross-lane permutes through the LDS crossbar.
// (row lanes only: WAVE_LOCAL lines, thread u of a line on lane u mod T)
template <int N, int E, int s, bool WAVE_LOCAL>
constexpr bool swap_exchange() {
  return WAVE_LOCAL && E == 16 && (N / E == 64 || N / E == 32) &&
         s + 1 < sched_stages(N, E) && sched_radix(N, E, s) == 16 && sched_ns(N, E, s) == 16;
}
__device__ __forceinline__ void swap32(float2& a, float2& b) {
  const auto rx = __builtin_amdgcn_permlane32_swap(__float_as_uint(a.x), __float_as_uint(b.x), false, false);
  const auto ry = __builtin_amdgcn_permlane32_swap(__float_as_uint(a.y), __float_as_uint(b.y), false, false);
  a = make_float2(__uint_as_float(rx[0]), __uint_as_float(ry[0]));
  b = make_float2(__uint_as_float(rx[1]), __uint_as_float(ry[1]));
}
__device__ __forceinline__ void swap16(float2& a, float2& b) {
  const auto rx = __builtin_amdgcn_permlane16_swap(__float_as_uint(a.x), __float_as_uint(b.x), false, false);
  const auto ry = __builtin_amdgcn_permlane16_swap(__float_as_uint(a.y), __float_as_uint(b.y), false, false);
  a = make_float2(__uint_as_float(rx[0]), __uint_as_float(ry[0]));
  b = make_float2(__uint_as_float(rx[1]), __uint_as_float(ry[1]));
}
// x: the 16 outputs of the thread's butterfly; v: the next stage's slots
template <int T>
__device__ __forceinline__ void swap_exchange_16(float2* x, float2* v) {
  if constexpr (T == 64) {
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if ((q & 2) == 0) swap32(x[q], x[q | 2]);  // lane bit 5 <-> register bit 1
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if ((q & 1) == 0) swap16(x[q], x[q | 1]);  // lane bit 4 <-> register bit 0
    // register r = (q/4, c): slot m = 4c + q/4
#pragma unroll
    for (int m = 0; m < 16; ++m) v[m] = x[((m & 3) << 2) | (m >> 2)];
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if ((q & 1) == 0) swap16(x[q], x[q | 1]);  // lane bit 4 <-> register bit 0
    // register r = (q/2, c): slot m = 8c + q/2
#pragma unroll
    for (int m = 0; m < 16; ++m) v[m] = x[((m & 7) << 1) | (m >> 3)];
  }
}

template <int N, int E, int S, bool WAVE_LOCAL, class Lds, bool SPLIT, int s, class LdsT, class TW>
__device__ __forceinline__ void run_stage(float2* v, LdsT* lds, const TW& tw, int u, int line) {
  static_assert(SPLIT == std::is_same<LdsT, float>::value, "LDS element type");
  constexpr int T = N / E;
  constexpr int NST = sched_stages(N, E);
  constexpr int R = sched_radix(N, E, s);
  constexpr int NS = sched_ns(N, E, s);
  constexpr int KB = E / R;
  static_assert(KB * R == E, "radix must divide the values per thread");
  constexpr bool last = (s == NST - 1);
  constexpr int OFF = sched_tw_off(N, E, s);
  static_for<0, KB>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    float2 x[R];
#pragma unroll
    for (int r = 0; r < R; ++r) x[r] = v[k + r * KB];
    const int b = u + T * k;
    const int j = b & (NS - 1);
    if constexpr (s > 0) {
#pragma unroll
      for (int r = 1; r < R; ++r) {
        x[r] = apply_tw<S>(x[r], tw_at<s>(tw, (uint32_t)(OFF + (r - 1) * NS), (uint32_t)j));
        // bound the twiddle loads in flight for large radices (VGPR budget)
        if constexpr (R > 16) {
          if ((r & 15) == 15) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    dft<R, S>(x);
    if constexpr (last || SPLIT) {
#pragma unroll
      for (int r = 0; r < R; ++r) v[k + r * KB] = x[r];
    } else if constexpr (swap_exchange<N, E, s, WAVE_LOCAL>()) {
      static_assert(WAVE_LOCAL && !SPLIT && KB == 1, "lane-swap exchange shape");
      swap_exchange_16<T>(x, v);
    } else {
      using I = StageIdx<T, R, NS, k>;
      const int base = I::base(u);
      static_for<0, R>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        lds[Lds::template at_k<I::K0 + r * NS, I::A>(line, base)] = x[r];
      });
    }
    // keep the scheduler from hoisting the next butterflies' twiddle loads
    // above this one: with many values per thread that would exhaust VGPRs
    if constexpr (KB > 1 && E > 16) __builtin_amdgcn_sched_barrier(0);
  });
  if constexpr (!last && !SPLIT && !swap_exchange<N, E, s, WAVE_LOCAL>()) {
    lds_sync<WAVE_LOCAL>();
    static_for<0, E>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      v[m] = lds[Lds::template at_k<T * m>(line, u)];
    });
    // the next stage writes LDS again (unless its exchange is a lane swap)
    if constexpr (s + 1 < NST - 1 && !swap_exchange<N, E, s + 1, WAVE_LOCAL>()) lds_sync<WAVE_LOCAL>();
  } else if constexpr (!last && SPLIT) {
    // real parts, then imaginary parts (v[.].y still hold the butterfly
    // outputs meanwhile).  For the second half the empty asm hides that the
    // indices are unchanged, so the LDS addresses are recomputed rather than
    // kept live across the barriers.
    auto exchange = [&](auto half, int uu, int ll) {
      constexpr bool IM = decltype(half)::value;
      static_for<0, KB>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        using I = StageIdx<T, R, NS, k>;
        const int base = I::base(uu);
        static_for<0, R>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          const float2 y = v[k + r * KB];
          lds[Lds::template at_k<I::K0 + r * NS, I::A>(ll, base)] = IM ? y.y : y.x;
        });
      });
      lds_sync<WAVE_LOCAL>();
      static_for<0, E>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        const float w = lds[Lds::template at_k<T * m>(ll, uu)];
        if constexpr (IM) v[m].y = w; else v[m].x = w;
      });
    };
    // Each half (and each stage) takes an opaque copy of the indices: the
    // read addresses are the same in every exchange, and kept live from one
    // exchange to the next they spilled (k_fs_cols<4096>: 6 VGPRs).
    int u1 = u, line1 = line;
    asm volatile("" : "+v"(u1), "+v"(line1));
    exchange(std::integral_constant<bool, false>{}, u1, line1);
    lds_sync<WAVE_LOCAL>();
    int u2 = u, line2 = line;
    asm volatile("" : "+v"(u2), "+v"(line2));
    exchange(std::integral_constant<bool, true>{}, u2, line2);
    if constexpr (s + 1 < NST - 1) lds_sync<WAVE_LOCAL>();
  }
}

template <int N, int E, int S, bool WAVE_LOCAL, class Lds, bool SPLIT, class LdsT, class TW>
__device__ __forceinline__ void run_stages(float2* v, LdsT* lds, const TW& tw, int u, int line) {
  static_for<0, sched_stages(N, E)>([&](auto sc) {
    run_stage<N, E, S, WAVE_LOCAL, Lds, SPLIT, decltype(sc)::value>(v, lds, tw, u, line);
  });
}

// Blocks are dispatched to the 8 XCDs of the chip round-robin by index, and
// each XCD has its own L2.  Renumber them so that the blocks one XCD runs at
// the same time handle adjacent line groups: their short strided runs then
// share L2 lines instead of being fetched separately by 8 XCDs.
__device__ __forceinline__ uint32_t xcd_grouped_block(uint32_t b, uint32_t nblocks) {
  const uint32_t full = nblocks & ~7u;
  if (b >= full) return b;
  return (b & 7u) * (full >> 3) + (b >> 3);
}


// Persistent passes whose workgroup holds a CU alone start in lockstep:
// every CU loads its first tile at once and then computes while HBM idles,
// and tiles of equal work keep them in step.  Half of each XCD's workgroups
// (blocks are dealt to the 8 XCDs round-robin, so index bit 3 halves each
// XCD's set) therefore start `ticks` of the constant-rate wall clock late,
// which puts the two halves' load and compute phases out of step for the
// rest of the launch.  The wait is bounded by the clock.
__device__ __forceinline__ void stagger_start(int64_t ticks) {
  if (ticks > 0 && ((blockIdx.x >> 3) & 1u)) {
    const long long t0 = wall_clock64();
    while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(4);
  }
}

}  // namespace fftamd
