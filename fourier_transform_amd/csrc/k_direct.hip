// Band-limited direct transforms of real rows, for any row length n: the
// direct trigonometric summation that the WGSL Fourier-stage source
// (turing-sphere fourier.ts, dftSynthWGSL / dftAnalysWGSL) offers beside its
// FFT, as a path for lengths the FFT does not take and as a cross-check.
//
// Both directions are one real matrix product over a batch of rows, run on
// the fp32 matrix cores (v_mfma_f32_32x32x2f32):
//   analysis   F[r][2m + h] = sum_j x[r][j] B[j][2m + h]
//              B[j][2m] = cos(2 pi mj/n), B[j][2m+1] = -sin(2 pi mj/n)
//   synthesis  x[r][j] = sum_{c < 2(mmax+1)} F[r][c] S[c][j]
//              S[2m][j] = w_m cos(2 pi mj/n), S[2m+1][j] = -w_m sin(2 pi mj/n),
//              w_0 = 1, w_m = 2 for m >= 1 (mmax < n/2)
// (F[r][c] is the float view of the complex spectrum: re at 2m, im at 2m+1).
// As in the source, no cos/sin is evaluated on the device: the factors come
// from e^{-2 pi i u/n}, u = 0..floor(n/2), computed on the host in f64 and
// rounded once, indexed by t = (m j) mod n folded to u = min(t, n - t).  The
// table sits in LDS; each lane generates the B operand it feeds to the matrix
// cores from it, keeping t incrementally (one add and a conditional subtract
// per step), so B never exists in memory.
//
// Tiling: a workgroup computes a 128 x 128 block of the result with four
// waves; wave w owns columns 32w..32w+31 and all 128 rows (four 32 x 32
// accumulators sharing one B operand per step).  The A operand (rows of x or
// of F) is staged in LDS 32 k-values at a time, the next slice prefetched into
// registers while the current one is consumed.  Within a slice, matrix-core
// step s takes k = s in lanes 0..31 and k = 16 + s in lanes 32..63, so each
// lane reads its A values as 16 contiguous floats.
//
// Accumulation is two-level: each 32-term slice is summed by the matrix cores
// into a fresh accumulator that is then added to the running total, so fp32
// rounding grows like sqrt(K/32) + sqrt(32) rather than sqrt(K).
#include "kernels.hpp"

namespace fftamd {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kDirBM = 128;  // rows (batch) per workgroup tile
constexpr int kDirBN = 128;  // columns per workgroup tile
constexpr int kDirBK = 32;   // k values per LDS slice
constexpr int kDirThreads = 256;
constexpr int kDirPitch = kDirBK + 4;  // floats per row of the A slice in LDS
constexpr int kDirectCUs = 256;       // compute units of the MI355X

__host__ __device__ constexpr int direct_table_floats(int n) { return (2 * (n / 2 + 1) + 3) & ~3; }
__host__ __device__ constexpr int direct_lds_bytes(int n) {
  return (direct_table_floats(n) + kDirBM * kDirPitch) * 4;
}

// A slice loader: 16 floats per thread.
//   analysis (SYN = false): x[r][k], VEC: n % 4 == 0 (float4 loads)
//   synthesis, row-major spectrum: F[r][m], VEC: (mmax + 1) even (float4 = 2 bins)
//   synthesis, m-major spectrum: F[m][r] (float2 loads, consecutive rows)
template <bool SYN, bool MMAJOR, bool VEC>
struct SliceIO {
  float v[16];
  __device__ __forceinline__ void load(const DirectArgs& a, int64_t row0, int k0, int tid) {
    const int64_t M = a.rows;
    if constexpr (!SYN && VEC) {
      const float* x = static_cast<const float*>(a.in);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid + kDirThreads * i, r = e >> 3, q = e & 7;
        const int64_t gr = row0 + r;
        const int gk = k0 + 4 * q;
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gr < M && gk < a.n) f = *reinterpret_cast<const float4*>(x + gr * a.n + gk);
        v[4 * i] = f.x, v[4 * i + 1] = f.y, v[4 * i + 2] = f.z, v[4 * i + 3] = f.w;
      }
    } else if constexpr (!SYN) {
      const float* x = static_cast<const float*>(a.in);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = tid + kDirThreads * i, r = e >> 5, k = e & 31;
        const int64_t gr = row0 + r;
        v[i] = (gr < M && k0 + k < a.n) ? x[gr * a.n + k0 + k] : 0.f;
      }
    } else if constexpr (!MMAJOR && VEC) {
      const float* F = static_cast<const float*>(a.in);
      const int nb = a.mmax + 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid + kDirThreads * i, r = e >> 3, q = e & 7;
        const int64_t gr = row0 + r;
        const int m = k0 / 2 + 2 * q;
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gr < M && m < nb) f = *reinterpret_cast<const float4*>(F + 2 * (gr * nb + m));
        v[4 * i] = f.x, v[4 * i + 1] = f.y, v[4 * i + 2] = f.z, v[4 * i + 3] = f.w;
      }
    } else {
      const float2* F = static_cast<const float2*>(a.in);
      const int nb = a.mmax + 1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = tid + kDirThreads * i;
        const int r = MMAJOR ? (e & 127) : (e >> 4), p = MMAJOR ? (e >> 7) : (e & 15);
        const int64_t gr = row0 + r;
        const int m = k0 / 2 + p;
        float2 f = make_float2(0.f, 0.f);
        if (gr < M && m < nb) f = MMAJOR ? F[(int64_t)m * M + gr] : F[gr * nb + m];
        v[2 * i] = f.x, v[2 * i + 1] = f.y;
      }
    }
  }
  __device__ __forceinline__ void store(float* As, int tid) const {
    if constexpr ((!SYN && VEC) || (SYN && !MMAJOR && VEC)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid + kDirThreads * i, r = e >> 3, q = e & 7;
        *reinterpret_cast<float4*>(As + r * kDirPitch + 4 * q) =
            make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
      }
    } else if constexpr (!SYN) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = tid + kDirThreads * i;
        As[(e >> 5) * kDirPitch + (e & 31)] = v[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = tid + kDirThreads * i;
        const int r = MMAJOR ? (e & 127) : (e >> 4), p = MMAJOR ? (e >> 7) : (e & 15);
        *reinterpret_cast<float2*>(As + r * kDirPitch + 2 * p) = make_float2(v[2 * i], v[2 * i + 1]);
      }
    }
  }
};

template <bool SYN, bool MMAJOR, bool VEC>
__global__ __launch_bounds__(kDirThreads) void k_direct(DirectArgs a) {
  extern __shared__ float4 smem4[];
  float* smem = reinterpret_cast<float*>(smem4);
  lds_poison_dynamic(smem, (uint32_t)direct_lds_bytes(a.n));
  const uint32_t n = (uint32_t)a.n, half = n / 2;
  float* T = smem;                                    // (cos, -sin)(2 pi u/n), u <= n/2
  float* As = smem + direct_table_floats((int)n);     // A slice [128][kDirPitch]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int64_t M = a.rows;
  const int nbins = a.mmax + 1;
  const int K = SYN ? 2 * nbins : (int)n;
  const int N = SYN ? (int)n : 2 * nbins;
  const uint32_t ntiles = (uint32_t)((N + kDirBN - 1) / kDirBN);
  const uint32_t b = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int64_t row0 = (int64_t)(b / ntiles) * kDirBM;
  const int col0 = (int)(b % ntiles) * kDirBN;
  const int col = col0 + wave * 32 + li;  // this lane's output column

  SliceIO<SYN, MMAJOR, VEC> io;
  io.load(a, row0, 0, tid);
  for (uint32_t u = tid; u <= half; u += kDirThreads)
    reinterpret_cast<float2*>(T)[u] = a.trig[u];
  io.store(As, tid);

  // table index state (see the header): analysis walks k with m fixed by the
  // column, synthesis walks m with j fixed by the column
  uint32_t t, inc, adv;
  int hp = 0;
  if (SYN) {
    const uint32_t jr = (uint32_t)col % n;
    t = (8u * h * jr) % n;        // m = 8h at the first slice
    inc = jr;                     // m + 1
    adv = (8u * jr) % n;          // m + 8 more at the end of a slice
  } else {
    const uint32_t mr = ((uint32_t)col >> 1) % n;
    hp = col & 1;
    t = (16u * h * mr) % n;       // k = 16h at the first slice
    inc = mr;                     // k + 1
    adv = (16u * mr) % n;         // k + 16 more at the end of a slice
  }
  auto step_t = [&](uint32_t d) {
    t += d;
    if (t >= n) t -= n;
  };

  v16f acc[4], zero;
#pragma unroll
  for (int v = 0; v < 16; ++v) zero[v] = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = zero;

  lds_barrier();
  for (int k0 = 0; k0 < K; k0 += kDirBK) {
    const bool more = k0 + kDirBK < K;
    if (more) io.load(a, row0, k0 + kDirBK, tid);
    v16f part[4];
    float2 bs = make_float2(0.f, 0.f);  // synthesis: (w cos, -w sin) of the current m
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      float4 av[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        av[q] = *reinterpret_cast<const float4*>(As + (32 * q + li) * kDirPitch + 16 * h + 4 * ch);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int s = 4 * ch + s4;
        const uint32_t u = t <= half ? t : n - t;
        const bool flip = t > half;
        float bv;
        if (SYN) {
          if ((s & 1) == 0) {
            const float2 e = reinterpret_cast<const float2*>(T)[u];
            const bool m0 = k0 == 0 && h == 0 && s == 0;
            bs.x = m0 ? 1.f : 2.f * e.x;
            bs.y = 2.f * (flip ? -e.y : e.y);
            bv = bs.x;
          } else {
            bv = bs.y;
            step_t(inc);
          }
        } else {
          const float e = T[2 * u + hp];
          bv = (hp && flip) ? -e : e;
          step_t(inc);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float avq = s4 == 0 ? av[q].x : s4 == 1 ? av[q].y : s4 == 2 ? av[q].z : av[q].w;
          part[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(avq, bv, s == 0 ? zero : part[q], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += part[q];
    step_t(adv);
    if (more) {
      lds_barrier();
      io.store(As, tid);
      lds_barrier();
    }
  }

  // store: accumulator q holds C[32q + i][j], j = lane % 32,
  // i = 8(v/4) + 4(lane/32) + v%4
  if (col >= N) return;
  float* o = static_cast<float*>(a.out);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t gr = row0 + 32 * q + 8 * (v >> 2) + 4 * h + (v & 3);
      if (gr >= M) continue;
      if (SYN)
        o[gr * (int64_t)n + col] = acc[q][v];
      else if (MMAJOR)
        o[(int64_t)(col >> 1) * 2 * M + 2 * gr + (col & 1)] = acc[q][v];
      else
        o[gr * 2 * nbins + col] = acc[q][v];
    }
  }
}

// ---------------------------------------------------------------------------
// Small problems (fewer than two 128 x 128 tiles per CU): workgroup tiles of
// 32 RB rows x 32 columns, the four waves splitting K (wave w takes the
// 32-value slices w, w + 4, ...), summed at the end through LDS in a fixed
// order.  A goes straight from memory to registers (lane (i, h) needs row i,
// k = 16h .. 16h + 15 of each slice), next slice prefetched.
// ---------------------------------------------------------------------------
template <bool SYN, bool MMAJOR, bool VEC, int RB>
struct LaneA {
  float v[RB][16];
  __device__ __forceinline__ void load(const DirectArgs& a, int64_t row0, int k0, int li, int h) {
    const int64_t M = a.rows;
    const int kb = k0 + 16 * h;
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int64_t gr = row0 + 32 * q + li;
      const bool rok = gr < M;
      if constexpr (!SYN && VEC) {
        const float* x = static_cast<const float*>(a.in) + gr * a.n;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
          if (rok && kb + 4 * c < a.n) f = *reinterpret_cast<const float4*>(x + kb + 4 * c);
          v[q][4 * c] = f.x, v[q][4 * c + 1] = f.y, v[q][4 * c + 2] = f.z, v[q][4 * c + 3] = f.w;
        }
      } else if constexpr (!SYN) {
        const float* x = static_cast<const float*>(a.in) + gr * a.n;
#pragma unroll
        for (int c = 0; c < 16; ++c) v[q][c] = (rok && kb + c < a.n) ? x[kb + c] : 0.f;
      } else if constexpr (!MMAJOR && VEC) {
        const int nb2 = 2 * (a.mmax + 1);
        const float* F = static_cast<const float*>(a.in) + gr * nb2;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
          if (rok && kb + 4 * c < nb2) f = *reinterpret_cast<const float4*>(F + kb + 4 * c);
          v[q][4 * c] = f.x, v[q][4 * c + 1] = f.y, v[q][4 * c + 2] = f.z, v[q][4 * c + 3] = f.w;
        }
      } else {
        const int nb = a.mmax + 1;
        const float2* F = static_cast<const float2*>(a.in);
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int m = kb / 2 + p;
          float2 f = make_float2(0.f, 0.f);
          if (rok && m < nb) f = MMAJOR ? F[(int64_t)m * M + gr] : F[gr * nb + m];
          v[q][2 * p] = f.x, v[q][2 * p + 1] = f.y;
        }
      }
    }
  }
};

template <bool SYN, bool MMAJOR, bool VEC, int RB>
__global__ __launch_bounds__(kDirThreads) void k_direct_small(DirectArgs a) {
  extern __shared__ float4 smem4[];
  float* smem = reinterpret_cast<float*>(smem4);
  lds_poison_dynamic(smem, (uint32_t)(direct_table_floats(a.n) + 4 * RB * 1024) * 4u);
  const uint32_t n = (uint32_t)a.n, half = n / 2;
  float* T = smem;
  float* red = smem + direct_table_floats((int)n);  // [4 waves][RB][16][64 lanes]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int64_t M = a.rows;
  const int nbins = a.mmax + 1;
  const int K = SYN ? 2 * nbins : (int)n;
  const int N = SYN ? (int)n : 2 * nbins;
  const uint32_t ntiles = (uint32_t)((N + 31) / 32);
  const uint32_t b = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int64_t row0 = (int64_t)(b / ntiles) * (32 * RB);
  const int col = (int)(b % ntiles) * 32 + li;

  for (uint32_t u = tid; u <= half; u += kDirThreads)
    reinterpret_cast<float2*>(T)[u] = a.trig[u];

  // table index state: slices w, w + 4, ... (see the big-tile kernel)
  uint32_t t, inc, adv;
  int hp = 0;
  if (SYN) {
    const uint32_t jr = (uint32_t)col % n;
    t = ((16u * wave + 8u * h) * jr) % n;   // m = 16w + 8h
    inc = jr;
    adv = (56u * jr) % n;                   // next slice: m + 64 in all
  } else {
    const uint32_t mr = ((uint32_t)col >> 1) % n;
    hp = col & 1;
    t = ((32u * wave + 16u * h) * mr) % n;  // k = 32w + 16h
    inc = mr;
    adv = (112u * mr) % n;                  // next slice: k + 128 in all
  }
  auto step_t = [&](uint32_t d) {
    t += d;
    if (t >= n) t -= n;
  };

  v16f acc[RB], zero;
#pragma unroll
  for (int v = 0; v < 16; ++v) zero[v] = 0.f;
#pragma unroll
  for (int q = 0; q < RB; ++q) acc[q] = zero;

  LaneA<SYN, MMAJOR, VEC, RB> cur, nxt;
  int k0 = 32 * wave;
  if (k0 < K) cur.load(a, row0, k0, li, h);
  lds_barrier();  // table ready
  for (; k0 < K; k0 += 128) {
    const bool more = k0 + 128 < K;
    if (more) nxt.load(a, row0, k0 + 128, li, h);
    v16f part[RB];
    float2 bs = make_float2(0.f, 0.f);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint32_t u = t <= half ? t : n - t;
      const bool flip = t > half;
      float bv;
      if (SYN) {
        if ((s & 1) == 0) {
          const float2 e = reinterpret_cast<const float2*>(T)[u];
          const bool m0 = k0 == 0 && h == 0 && s == 0;
          bs.x = m0 ? 1.f : 2.f * e.x;
          bs.y = 2.f * (flip ? -e.y : e.y);
          bv = bs.x;
        } else {
          bv = bs.y;
          step_t(inc);
        }
      } else {
        const float e = T[2 * u + hp];
        bv = (hp && flip) ? -e : e;
        step_t(inc);
      }
#pragma unroll
      for (int q = 0; q < RB; ++q)
        part[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(cur.v[q][s], bv, s == 0 ? zero : part[q], 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < RB; ++q) acc[q] += part[q];
    step_t(adv);
    if (more) cur = nxt;
  }

  // fixed-order sum of the four waves' partial results
#pragma unroll
  for (int q = 0; q < RB; ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[((wave * RB + q) * 16 + v) * 64 + lane] = acc[q][v];
  lds_barrier();
  float* o = static_cast<float*>(a.out);
#pragma unroll
  for (int i = 0; i < RB * 4; ++i) {
    const int e = tid + kDirThreads * i;  // (q, v, lane) of wave 0's layout
    const int q = e >> 10, v = (e >> 6) & 15, l = e & 63;
    float sum = red[e];
#pragma unroll
    for (int w = 1; w < 4; ++w) sum += red[w * RB * 1024 + e];
    const int c = (int)(b % ntiles) * 32 + (l & 31);
    const int64_t gr = row0 + 32 * q + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
    if (c >= N || gr >= M) continue;
    if (SYN)
      o[gr * (int64_t)n + c] = sum;
    else if (MMAJOR)
      o[(int64_t)(c >> 1) * 2 * M + 2 * gr + (c & 1)] = sum;
    else
      o[gr * 2 * nbins + c] = sum;
  }
}

template <bool SYN>
hipError_t launch_direct_as(const DirectArgs& a, hipStream_t st, int64_t N, bool in16) {
  const int64_t big = ((a.rows + kDirBM - 1) / kDirBM) * ((N + kDirBN - 1) / kDirBN);
  const bool vec = SYN ? (a.mmax + 1) % 2 == 0 && in16 : a.n % 4 == 0 && in16;
  const dim3 block(kDirThreads);
  if (big >= 2 * kDirectCUs) {
    const size_t lds = (size_t)direct_lds_bytes(a.n);
    if (big > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)big);
    if (a.mmajor && (SYN || !vec))
      FFTAMD_LAUNCH((k_direct<SYN, true, false>), grid, block, lds, st, a);
    else if (a.mmajor)
      FFTAMD_LAUNCH((k_direct<SYN, true, true>), grid, block, lds, st, a);
    else if (vec)
      FFTAMD_LAUNCH((k_direct<SYN, false, true>), grid, block, lds, st, a);
    else
      FFTAMD_LAUNCH((k_direct<SYN, false, false>), grid, block, lds, st, a);
  } else {
    constexpr int RB = 1;
    const int64_t blocks = ((a.rows + 32 * RB - 1) / (32 * RB)) * ((N + 31) / 32);
    const size_t lds = (size_t)(direct_table_floats(a.n) + 4 * RB * 1024) * 4;
    const dim3 grid((uint32_t)blocks);
    if (a.mmajor && (SYN || !vec))
      FFTAMD_LAUNCH((k_direct_small<SYN, true, false, RB>), grid, block, lds, st, a);
    else if (a.mmajor)
      FFTAMD_LAUNCH((k_direct_small<SYN, true, true, RB>), grid, block, lds, st, a);
    else if (vec)
      FFTAMD_LAUNCH((k_direct_small<SYN, false, true, RB>), grid, block, lds, st, a);
    else
      FFTAMD_LAUNCH((k_direct_small<SYN, false, false, RB>), grid, block, lds, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_direct(bool synthesis, const DirectArgs& a, hipStream_t st) {
  if (a.n < 2 || a.n > kMaxDirectLength || a.mmax < 0 || 2 * (int64_t)a.mmax >= a.n || a.rows < 1)
    return hipErrorInvalidValue;
  const bool in16 = ((uintptr_t)a.in & 15) == 0;  // float4 loads need 16-byte alignment
  if (synthesis) return launch_direct_as<true>(a, st, a.n, in16);
  return launch_direct_as<false>(a, st, 2 * (int64_t)(a.mmax + 1), in16);
}

}  // namespace fftamd
