// Element-wise kernels around an any-length complex transform, for real
// transforms whose length is not a power of two.
//
// Even n = 2h follows the WGSL Fourier-stage source (turing-sphere
// fourier.ts, header comment, fftAnalysRealWGSL / fftSynthRealWGSL): the real
// row is read as h complex values z_m = x_{2m} + i x_{2m+1}, transformed with
// length h, and split by the even/odd symmetry,
//   X_k = Xe + e^{-2 pi i k/n} Xo,  Xe = (Z_k + conj Z_{h-k})/2,
//   Xo = -i (Z_k - conj Z_{h-k})/2,  Z_h = Z_0;
// synthesis assembles Z_k = (X_k + conj X_{h-k}) + i e^{+2 pi i k/n}
// (X_k - conj X_{h-k}) and the inverse transform of length h gives x as h
// complex values.  Odd n uses the definition directly: the forward transform
// of (x, 0) keeps bins 0..mmax, and synthesis inverts the full Hermitian
// spectrum (X_0 = Re F_0, X_m = F_m, X_{n-m} = conj F_m) and keeps the real
// part.  Bins above mmax are zero; Im F_0 (and Im F_h when mmax = h) is
// ignored.
//
// Work items are (row, bin) pairs; with the m-major spectrum consecutive
// threads take consecutive rows, so the spectrum side is the coalesced one.
#include "kernels.hpp"

namespace fftamd {

namespace {
constexpr int kRealAnyThreads = 256;

// (row, bin) of work item t: bins fastest (row-major spectrum) or rows
// fastest (m-major).  One division by the selected extent, then value
// selects (selecting between two output pointers put them in scratch).
__device__ __forceinline__ void item(const RealAnyArgs& a, int64_t t, int64_t nk, int64_t* row, int64_t* k) {
  const int64_t d = a.mmajor ? a.rows : nk;
  const int64_t q = t / d, r = t - q * d;
  *row = a.mmajor ? r : q;
  *k = a.mmajor ? q : r;
}
__device__ __forceinline__ int64_t spec_at(const RealAnyArgs& a, int64_t row, int64_t k) {
  return a.mmajor ? k * a.rows + row : row * (a.mmax + 1) + k;
}
// X_k of the band-limited Hermitian spectrum held as bins 0..mmax
__device__ __forceinline__ float2 bin(const RealAnyArgs& a, const float2* F, int64_t row, int64_t k) {
  if (k > a.mmax) return make_float2(0.f, 0.f);
  const float2 v = F[spec_at(a, row, k)];
  if (k == 0 || 2 * k == a.n) return make_float2(v.x, 0.f);
  return v;
}

__global__ __launch_bounds__(kRealAnyThreads) void k_real_unpack(RealAnyArgs a) {
  const int64_t nk = a.mmax + 1, total = a.rows * nk;
  const int64_t t = (int64_t)blockIdx.x * kRealAnyThreads + threadIdx.x;
  if (t >= total) return;
  int64_t row, k;
  item(a, t, nk, &row, &k);
  const int64_t h = a.len;
  const float2* Z = static_cast<const float2*>(a.in) + row * h;
  const float2 zk = Z[k % h];
  const float2 zh = Z[(h - k) % h];
  const float2 xe = make_float2(0.5f * (zk.x + zh.x), 0.5f * (zk.y - zh.y));
  const float2 d = make_float2(0.5f * (zk.x - zh.x), 0.5f * (zk.y + zh.y));
  const float2 xo = make_float2(d.y, -d.x);
  static_cast<float2*>(a.out)[spec_at(a, row, k)] = cadd(xe, cmul(xo, a.rt[k]));
}

__global__ __launch_bounds__(kRealAnyThreads) void k_real_pack(RealAnyArgs a) {
  const int64_t h = a.len, total = a.rows * h;
  const int64_t t = (int64_t)blockIdx.x * kRealAnyThreads + threadIdx.x;
  if (t >= total) return;
  int64_t row, k;
  // Z is written row-major; with the m-major spectrum walk rows fastest
  if (a.mmajor) {
    k = t / a.rows;
    row = t - k * a.rows;
  } else {
    row = t / h;
    k = t - row * h;
  }
  const float2* F = static_cast<const float2*>(a.in);
  const float2 xk = bin(a, F, row, k);
  const float2 xh = bin(a, F, row, h - k);  // h - k in 1..h
  const float2 cj = cconj(xh);
  const float2 s = cadd(xk, cj);
  const float2 b = cmulc(csub(xk, cj), a.rt[k]);  // times e^{+2 pi i k/n}
  static_cast<float2*>(a.out)[row * h + k] = make_float2(s.x - b.y, s.y + b.x);
}

__global__ __launch_bounds__(kRealAnyThreads) void k_real_complexify(RealAnyArgs a) {
  const int64_t total = a.rows * (int64_t)a.n;
  const int64_t t = (int64_t)blockIdx.x * kRealAnyThreads + threadIdx.x;
  if (t >= total) return;
  static_cast<float2*>(a.out)[t] = make_float2(static_cast<const float*>(a.in)[t], 0.f);
}

__global__ __launch_bounds__(kRealAnyThreads) void k_real_extract(RealAnyArgs a) {
  const int64_t nk = a.mmax + 1, total = a.rows * nk;
  const int64_t t = (int64_t)blockIdx.x * kRealAnyThreads + threadIdx.x;
  if (t >= total) return;
  int64_t row, k;
  item(a, t, nk, &row, &k);
  static_cast<float2*>(a.out)[spec_at(a, row, k)] = static_cast<const float2*>(a.in)[row * a.n + k];
}

__global__ __launch_bounds__(kRealAnyThreads) void k_real_hermitian(RealAnyArgs a) {
  const int64_t n = a.n, total = a.rows * n;
  const int64_t t = (int64_t)blockIdx.x * kRealAnyThreads + threadIdx.x;
  if (t >= total) return;
  int64_t row, k;
  if (a.mmajor) {
    k = t / a.rows;
    row = t - k * a.rows;
  } else {
    row = t / n;
    k = t - row * n;
  }
  const float2* F = static_cast<const float2*>(a.in);
  float2 v;
  if (k <= n / 2)
    v = bin(a, F, row, k);
  else
    v = cconj(bin(a, F, row, n - k));
  static_cast<float2*>(a.out)[row * n + k] = v;
}

__global__ __launch_bounds__(kRealAnyThreads) void k_real_part(RealAnyArgs a) {
  const int64_t total = a.rows * (int64_t)a.n;
  const int64_t t = (int64_t)blockIdx.x * kRealAnyThreads + threadIdx.x;
  if (t >= total) return;
  static_cast<float*>(a.out)[t] = static_cast<const float2*>(a.in)[t].x;
}

hipError_t launch_items(void (*k)(RealAnyArgs), int64_t total, const RealAnyArgs& a, hipStream_t st) {
  uint32_t grid;
  hipError_t e = grid_of(total, kRealAnyThreads, &grid);
  if (e != hipSuccess) return e;
  FFTAMD_LAUNCH(k, dim3(grid), dim3(kRealAnyThreads), 0, st, a);
  return hipGetLastError();
}
bool args_ok(const RealAnyArgs& a) {
  return a.rows >= 1 && a.n >= 3 && a.mmax >= 0 && 2 * (int64_t)a.mmax <= a.n && a.len >= 1;
}
}  // namespace

hipError_t launch_real_unpack(const RealAnyArgs& a, hipStream_t st) {
  if (!args_ok(a) || 2 * a.len != a.n) return hipErrorInvalidValue;
  return launch_items(k_real_unpack, a.rows * (a.mmax + 1), a, st);
}
hipError_t launch_real_pack(const RealAnyArgs& a, hipStream_t st) {
  if (!args_ok(a) || 2 * a.len != a.n) return hipErrorInvalidValue;
  return launch_items(k_real_pack, a.rows * a.len, a, st);
}
hipError_t launch_real_complexify(const RealAnyArgs& a, hipStream_t st) {
  if (!args_ok(a) || a.len != a.n) return hipErrorInvalidValue;
  return launch_items(k_real_complexify, a.rows * a.n, a, st);
}
hipError_t launch_real_extract(const RealAnyArgs& a, hipStream_t st) {
  if (!args_ok(a) || a.len != a.n) return hipErrorInvalidValue;
  return launch_items(k_real_extract, a.rows * (a.mmax + 1), a, st);
}
hipError_t launch_real_hermitian(const RealAnyArgs& a, hipStream_t st) {
  if (!args_ok(a) || a.len != a.n) return hipErrorInvalidValue;
  return launch_items(k_real_hermitian, a.rows * a.n, a, st);
}
hipError_t launch_real_part(const RealAnyArgs& a, hipStream_t st) {
  if (!args_ok(a) || a.len != a.n) return hipErrorInvalidValue;
  return launch_items(k_real_part, a.rows * a.n, a, st);
}

}  // namespace fftamd
