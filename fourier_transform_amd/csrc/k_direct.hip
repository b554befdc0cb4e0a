// Band-limited direct transforms of real rows, for any row length n: the
// direct trigonometric summation that the WGSL Fourier-stage source
// (turing-sphere fourier.ts, dftSynthWGSL / dftAnalysWGSL) offers beside its
// FFT, as a path for lengths the FFT does not take and as a cross-check.
//
// Both directions are one real matrix product per batch of rows, run on the
// fp32 matrix cores (v_mfma_f32_32x32x2f32):
//   analysis   F[r][2m + h] = sum_j x[r][j] B[j][2m + h]
//              B[j][2m] = cos(2 pi mj/n), B[j][2m+1] = -sin(2 pi mj/n)
//   synthesis  x[r][j] = sum_{c < 2(mmax+1)} F[r][c] S[c][j]
//              S[2m][j] = w_m cos(2 pi mj/n), S[2m+1][j] = -w_m sin(2 pi mj/n),
//              w_0 = 1, w_m = 2 for m >= 1 (mmax < n/2)
// (F[r][c] is the float view of the complex spectrum: re at 2m, im at 2m+1).
// As in the source, the cos/sin factors are never evaluated on the device:
// they come from the plan's table trig[t] = (cos, sin)(2 pi t/n), computed on
// the host in f64 and rounded once, indexed by (m j) mod n.  Each thread keeps
// its table indices incrementally from one k tile to the next.
//
// Accumulation is two-level: each k tile (32 terms) is summed by the matrix
// cores into a fresh accumulator that is then added to the running total, so
// the fp32 rounding error grows with sqrt(K/32) + sqrt(32) rather than sqrt(K).
#include "kernels.hpp"

namespace fftamd {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kDirBM = 64;  // rows (batch) per tile
constexpr int kDirBN = 64;  // columns per tile
constexpr int kDirBK = 32;  // k depth staged in LDS per step
constexpr int kDirThreads = 256;
constexpr int kDirPad = 4;

// SYN: synthesis (spectrum -> rows), else analysis (rows -> spectrum).
// MMAJOR: spectrum stored [mmax+1][rows], else [rows][mmax+1] (complex).
template <bool SYN, bool MMAJOR>
__global__ __launch_bounds__(kDirThreads) void k_direct(DirectArgs a) {
  __shared__ float As[kDirBK][kDirBM + kDirPad];  // A tile, k-major
  __shared__ float Bs[kDirBK][kDirBN + kDirPad];  // B tile, k-major

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t M = a.rows;
  const uint32_t n = (uint32_t)a.n;
  const int mmax = a.mmax, nbins = mmax + 1;
  const int K = SYN ? 2 * nbins : (int)n;
  const int64_t row0 = (int64_t)blockIdx.x * kDirBM;
  const int col0 = blockIdx.y * kDirBN;
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;

  // table indices of this thread's four B entries, advanced per k tile
  uint32_t t[4], step;
  if (SYN) {  // entries (m = mr + 4i, j = col0 + (tid & 63)); m moves by 16 per tile
    const uint32_t j = (uint32_t)(col0 + (tid & 63)), mr = (uint32_t)(tid >> 6);
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = ((mr + 4u * i) * j) % n;
    step = ((uint32_t)(kDirBK / 2) * j) % n;
  } else {  // entries (j = jr + 8i, m = col0/2 + (tid & 31)); j moves by 32 per tile
    const uint32_t m = (uint32_t)(col0 / 2 + (tid & 31)), jr = (uint32_t)(tid >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = ((jr + 8u * i) * m) % n;
    step = ((uint32_t)kDirBK * m) % n;
  }

  v16f acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;

  for (int k0 = 0; k0 < K; k0 += kDirBK) {
    // ---- stage A (BM x BK), zero outside the matrix ----
    if (SYN) {
      const float2* F = static_cast<const float2*>(a.in);
#pragma unroll
      for (int i = 0; i < kDirBM * kDirBK / 2 / kDirThreads; ++i) {
        const int e = tid + kDirThreads * i;
        const int p = MMAJOR ? e / kDirBM : e % (kDirBK / 2);
        const int r = MMAJOR ? e % kDirBM : e / (kDirBK / 2);
        const int m = k0 / 2 + p;
        const int64_t gr = row0 + r;
        float2 v = make_float2(0.f, 0.f);
        if (gr < M && m < nbins) v = MMAJOR ? F[(int64_t)m * M + gr] : F[gr * nbins + m];
        As[2 * p][r] = v.x;
        As[2 * p + 1][r] = v.y;
      }
    } else {
      const float* x = static_cast<const float*>(a.in);
#pragma unroll
      for (int i = 0; i < kDirBM * kDirBK / kDirThreads; ++i) {
        const int e = tid + kDirThreads * i;
        const int k = e % kDirBK, r = e / kDirBK;
        const int64_t gr = row0 + r;
        const int gk = k0 + k;
        As[k][r] = (gr < M && gk < K) ? x[gr * (int64_t)n + gk] : 0.f;
      }
    }
    // ---- stage B from the table ----
    if (SYN) {
      const int jj = tid & 63, mr = tid >> 6;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ml = mr + 4 * i;
        const float w = (k0 == 0 && ml == 0) ? 1.f : 2.f;
        const float2 cs = a.trig[t[i]];
        Bs[2 * ml][jj] = w * cs.x;
        Bs[2 * ml + 1][jj] = -w * cs.y;
        t[i] += step;
        if (t[i] >= n) t[i] -= n;
      }
    } else {
      const int mi = tid & 31, jr = tid >> 5;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 cs = a.trig[t[i]];
        *reinterpret_cast<float2*>(&Bs[jr + 8 * i][2 * mi]) = make_float2(cs.x, -cs.y);
        t[i] += step;
        if (t[i] >= n) t[i] -= n;
      }
    }
    lds_barrier();
    // ---- 16 matrix-core steps over this tile, into a fresh accumulator ----
    v16f part;
#pragma unroll
    for (int v = 0; v < 16; ++v) part[v] = 0.f;
#pragma unroll
    for (int kk = 0; kk < kDirBK; kk += 2) {
      // lane: A[i][kk + lane/32] with i = lane % 32; B[kk + lane/32][j] with j = lane % 32
      const float av = As[kk + (lane >> 5)][wr + (lane & 31)];
      const float bv = Bs[kk + (lane >> 5)][wc + (lane & 31)];
      part = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, part, 0, 0, 0);
    }
    acc += part;
    lds_barrier();
  }

  // ---- store: lane holds C[i][j], j = lane % 32, i = 8(v/4) + 4(lane/32) + v%4 ----
  const int gc = col0 + wc + (lane & 31);
  const int N = SYN ? (int)n : 2 * nbins;
  if (gc >= N) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t gr = row0 + wr + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (gr >= M) continue;
    float* o = static_cast<float*>(a.out);
    if (SYN)
      o[gr * (int64_t)n + gc] = acc[v];
    else if (MMAJOR)
      o[(int64_t)(gc >> 1) * 2 * M + 2 * gr + (gc & 1)] = acc[v];
    else
      o[gr * 2 * nbins + gc] = acc[v];
  }
}

hipError_t launch_direct(bool synthesis, const DirectArgs& a, hipStream_t st) {
  if (a.n < 2 || a.n > kMaxDirectLength || a.mmax < 0 || 2 * (int64_t)a.mmax >= a.n || a.rows < 1)
    return hipErrorInvalidValue;
  const int64_t N = synthesis ? a.n : 2 * (int64_t)(a.mmax + 1);
  const int64_t gx = (a.rows + kDirBM - 1) / kDirBM, gy = (N + kDirBN - 1) / kDirBN;
  if (gx > 0x7fffffffLL || gy > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid((uint32_t)gx, (uint32_t)gy), block(kDirThreads);
  if (synthesis) {
    if (a.mmajor)
      hipLaunchKernelGGL((k_direct<true, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((k_direct<true, false>), grid, block, 0, st, a);
  } else {
    if (a.mmajor)
      hipLaunchKernelGGL((k_direct<false, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((k_direct<false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace fftamd
