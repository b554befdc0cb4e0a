// plan.cpp -- the C ABI of include/fft.h: argument checks, plan construction
// (path choice, host-f64 twiddle tables, scratch) and the launch sequence.
//
// Every argument check runs on the host before the first HIP call, so each
// error path can be exercised without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <complex>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <functional>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "fft.h"
#include "launch.hpp"
#include "shapes.hpp"
#include "stockham.hpp"

using namespace fftamd;

hipEvent_t& fftamd::exec_done_event() {
  thread_local hipEvent_t e = nullptr;
  return e;
}

namespace {

constexpr int kFourStepMaxLog = 2 * ilog2c(kMaxSinglePass);  // 2^28
// 2D images with at least this many rows split their column transform in two
// steps (64 x ny/64), each with long runs (see ColStageArgs)
constexpr int64_t kTallRows = 8192;
// longest mixed-radix convolution the one-kernel chirp transform searches
// (its measured gains were for n <= 4096, c <= 8192)
constexpr int64_t kMaxChirpMixedLength = 8192;
constexpr int kTallSplit = 64;
constexpr double kTwoPi = 6.283185307179586476925286766559;

// ---------------------------------------------------------------------------
// thread-local error state
// ---------------------------------------------------------------------------
struct ErrorState {
  int code = FFT_OK;
  std::string msg = "ok";
};
thread_local ErrorState g_err;

int set_err(int code, const std::string& msg) {
  g_err.code = code;
  g_err.msg = msg;
  return code;
}
int ok() { return set_err(FFT_OK, "ok"); }
int hip_err(hipError_t e, const char* what) {
  return set_err(e == hipErrorOutOfMemory ? FFT_ENOMEM : FFT_EHIP,
                 std::string(what) + ": " + hipGetErrorString(e));
}

bool is_pow2(int64_t n) { return n >= 1 && (n & (n - 1)) == 0; }

// ---------------------------------------------------------------------------
// twiddle tables, computed in f64 and rounded once to fp32 (round to nearest)
// ---------------------------------------------------------------------------
float2 root(int64_t e, int64_t len) {  // e^{-2 pi i e/len}, 0 <= e < len
  const double a = kTwoPi * (double)e / (double)len;
  return make_float2((float)std::cos(a), (float)-std::sin(a));
}

// stage table of the radix schedule for length n with e values per thread
// (layout: stockham.hpp, run_stage)
void append_stage_table(int n, int e, std::vector<float2>& t) {
  const int stages = sched_stages(n, e);
  for (int s = 1; s < stages; ++s) {
    const int R = sched_radix(n, e, s), NS = sched_ns(n, e, s);
    for (int r = 1; r < R; ++r)
      for (int j = 0; j < NS; ++j) t.push_back(root((int64_t)r * j, (int64_t)NS * R));
  }
  if (t.empty()) t.push_back(make_float2(1.f, 0.f));  // keep offsets valid
}

// Bluestein chirp e^{sign pi i q/n} for the integer exponent q, reduced
// modulo 2n first so that the angle is exact up to one rounding
float2 chirp(int64_t q, int64_t n, int sign) {
  const int64_t r = ((q % (2 * n)) + 2 * n) % (2 * n);
  const double a = kTwoPi * 0.5 * (double)r / (double)n;
  return make_float2((float)std::cos(a), (float)(sign * std::sin(a)));
}

// forward transform (e^{-2 pi i jk/m}) of a power-of-two length in f64 on the
// host, for plan tables only: iterative radix 2, every twiddle from cos/sin
// of its own angle
void host_fft_f64(std::vector<std::complex<double>>& a) {
  const size_t m = a.size();
  for (size_t i = 1, j = 0; i < m; ++i) {
    size_t bit = m >> 1;
    for (; j & bit; bit >>= 1) j ^= bit;
    j ^= bit;
    if (i < j) std::swap(a[i], a[j]);
  }
  for (size_t len = 2; len <= m; len <<= 1) {
    for (size_t k = 0; k < len / 2; ++k) {
      const double ang = -kTwoPi * (double)k / (double)len;
      const std::complex<double> w(std::cos(ang), std::sin(ang));
      for (size_t i = 0; i < m; i += len) {
        const std::complex<double> t = w * a[i + k + len / 2];
        a[i + k + len / 2] = a[i + k] - t;
        a[i + k] += t;
      }
    }
  }
}

// forward transform (e^{-2 pi i jk/m}) of any length in f64 on the host, for
// plan tables only: split by the smallest prime factor q of m (inputs q
// apart), recursively; a prime length is summed directly, every factor from
// cos/sin of its own angle (the product jk reduced mod m in integers)
void host_dft_f64(std::vector<std::complex<double>>& a) {
  const size_t m = a.size();
  if (m <= 1) return;
  size_t q = 2;
  while (m % q) ++q;
  std::vector<std::complex<double>> out(m);
  auto w = [m](size_t e) {
    const double ang = -kTwoPi * (double)(e % m) / (double)m;
    return std::complex<double>(std::cos(ang), std::sin(ang));
  };
  if (q == m) {
    for (size_t k = 0; k < m; ++k) {
      std::complex<double> s = 0.0;
      for (size_t j = 0; j < m; ++j) s += a[j] * w(j * k);
      out[k] = s;
    }
  } else {
    const size_t r = m / q;
    std::vector<std::vector<std::complex<double>>> sub(q, std::vector<std::complex<double>>(r));
    for (size_t i = 0; i < q; ++i)
      for (size_t j = 0; j < r; ++j) sub[i][j] = a[i + q * j];
    for (auto& v : sub) host_dft_f64(v);
    for (size_t k = 0; k < m; ++k) {
      std::complex<double> s = 0.0;
      for (size_t i = 0; i < q; ++i) s += w(i * k) * sub[i][k % r];
      out[k] = s;
    }
  }
  a.swap(out);
}

bool is_prime(int64_t n) {
  if (n < 2) return false;
  for (int64_t d = 2; d * d <= n; ++d)
    if (n % d == 0) return false;
  return true;
}

int64_t pow_mod(int64_t b, int64_t e, int64_t m) {
  int64_t r = 1 % m;
  b %= m;
  for (; e; e >>= 1, b = b * b % m)
    if (e & 1) r = r * b % m;
  return r;
}

// smallest generator of the nonzero residues mod a prime p
int64_t primitive_root(int64_t p) {
  std::vector<int64_t> qs;
  int64_t m = p - 1;
  for (int64_t d = 2; d * d <= m; ++d)
    if (m % d == 0) {
      qs.push_back(d);
      while (m % d == 0) m /= d;
    }
  if (m > 1) qs.push_back(m);
  for (int64_t g = 2; g < p; ++g) {
    bool gen = true;
    for (int64_t q : qs) gen = gen && pow_mod(g, (p - 1) / q, p) != 1;
    if (gen) return g;
  }
  return 1;  // p = 2
}

}  // namespace

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------
struct fft_plan {
  int dims = 1;
  int64_t n = 0, ny = 1, nx = 0, batch = 0;
  int kind = FFT_C2C, sign = FFT_FORWARD;
  int shift = 0;
  int64_t mmax = 0;
  int spec_layout = 0;
  int real_pairs = 0;
  bool executed = false;
  bool fourstep = false;
  int device = 0;
  // four-step split n = n1 * n2
  int n1 = 0, n2 = 0, bits = 0;
  // device resources
  float2* tables = nullptr;
  const float2* tw_a = nullptr;  // rows: n (1D), nx (2D), h (real), n1 (four-step rows)
  const float2* tw_b = nullptr;  // cols: ny (2D), n2 (four-step cols)
  const float2* rt = nullptr;    // real transforms: e^{-2 pi i k/n}, k = 0..n/2
  const float2* tw_full = nullptr;  // real transforms, pair mode: stage table for n
  const float2* thi = nullptr;
  const float2* tlo = nullptr;
  // 2D images through a scratch (8192 rows and more, and the 4096-row images
  // of the two-pass form): column steps A (length ny/64) and B (length 64),
  // W_ny table; fold: the two-pass form instead (tw_ca: rows of nx for the
  // fold kernel, tw_cb: the 2048-point columns)
  bool tall = false;
  bool fold = false;
  const float2* tw_ca = nullptr;
  const float2* tw_cb = nullptr;
  const float2* wt = nullptr;
  const float2* trig = nullptr;  // direct kinds: e^{-2 pi i u/n}, u = 0..n/2
  // C2C lengths that are not powers of two (Bluestein): transform length bm,
  // chirps c_j (and c_j times the shift ramp), forward transform of the chirp
  bool bluestein = false;
  bool bmixed = false;  // convolution length bm with a mixed-radix schedule (mx)
  int bm = 0;
  const float2* chirp = nullptr;
  const float2* chirp_shift = nullptr;
  const float2* chirp_ishift = nullptr;
  const float2* bhat = nullptr;
  const float2* bhat_t = nullptr;  // above m = 16384: bhat[k2 + n2*k1] at k2*n1 + k1
  // C2C lengths with no prime factor above 13 (mixed radix): the schedule, and
  // the load factors of the two shifts
  bool mixed = false;
  // C2C lengths with no prime factor above 13 that no one-kernel schedule
  // takes: the four-step n = n1 * n2 (n1, n2, bits, thi, tlo as above): the
  // n2-point column transforms (inner2's schedule) times W_n^{j1 k2} into
  // the scratch, the n1-point row plan (inner) in place there, and a
  // transpose to natural order that also applies the shift (a rotation)
  bool fsany = false;
  bool fs2 = false;  // two passes: inner holds the schedule of n1 for row tiles stored transposed
  bool rader = false;  // mx holds the schedule of n - 1
  MixedArgs mx{};
  const float2* rd_conv = nullptr;
  const float2* rd_perm = nullptr;  // int2 pairs (RaderArgs.perm) in float2 slots
  const float2* mx_shift = nullptr;
  const float2* mx_ishift = nullptr;
  // R2C/C2R of lengths that are not powers of two: an any-length C2C plan of
  // length n/2 (even n) or n (odd n) plus the packing kernels
  bool real_any = false;
  fft_plan* inner = nullptr;
  // 2D plans with an axis that is not a power of two: row plans of nx (inner)
  // and of ny (inner2, run on the transposed image)
  bool any2d = false;
  // column pass of those plans: 0 = transpose, row plan of ny, transpose
  // back (four HBM passes with the rows); 1 = k_c2c_cols in place (ny a power
  // of two, tw_b its table); 2 = k_mixed_cols in place (ny has a mixed-radix
  // schedule, inner2 holds it)
  int cols2d = 0;
  fft_plan* inner2 = nullptr;
  float2* scratch = nullptr;
  size_t scratch_bytes = 0;
  // completion of the plan's last exec outside graph capture (destroy waits
  // for it; an exec on another stream first waits for it)
  hipEvent_t done = nullptr;
  bool recorded = false;
  hipStream_t last_stream = nullptr;
};

namespace {

bool is_direct(int kind) { return kind == FFT_R2C_DIRECT || kind == FFT_C2R_DIRECT; }
bool is_analysis(int kind) { return kind == FFT_R2C || kind == FFT_R2C_DIRECT; }

int check_kind_sign(int kind, int sign) {
  if (kind < FFT_C2C || kind > FFT_C2R_DIRECT)
    return set_err(FFT_EINVAL, "kind must be FFT_C2C, FFT_R2C, FFT_C2R, FFT_R2C_DIRECT or FFT_C2R_DIRECT");
  if (sign != FFT_FORWARD && sign != FFT_INVERSE)
    return set_err(FFT_EINVAL, "sign must be FFT_FORWARD (-1) or FFT_INVERSE (+1)");
  if (is_analysis(kind) && sign != FFT_FORWARD)
    return set_err(FFT_EINVAL, "R2C kinds are forward transforms (sign must be -1)");
  if (kind != FFT_C2C && !is_analysis(kind) && sign != FFT_INVERSE)
    return set_err(FFT_EINVAL, "C2R kinds are inverse transforms (sign must be +1)");
  return FFT_OK;
}

int check_total(int64_t a, int64_t b, int64_t c) {
  // a*b*c*8 bytes must fit in int64
  const int64_t lim = INT64_MAX / 8;
  if (a > lim / b || a * b > lim / c) return set_err(FFT_EINVAL, "transform size overflows");
  return FFT_OK;
}

void free_plan(fft_plan* p) {
  if (!p) return;
  if (p->inner) free_plan(p->inner);
  if (p->inner2) free_plan(p->inner2);
  // returned in stream order on the null stream (see finish_plan)
  if (p->tables) (void)hipFreeAsync(p->tables, nullptr);
  if (p->scratch) (void)hipFreeAsync(p->scratch, nullptr);
  if (p->done) (void)hipEventDestroy(p->done);
  delete p;
}

// wait for the last recorded exec of the plan and of its inner plans (an
// inner plan records its own event, and the outer exec may have failed after
// the inner one was enqueued)
void wait_plan(fft_plan* p) {
  if (!p) return;
  if (p->recorded) (void)hipEventSynchronize(p->done);
  wait_plan(p->inner);
  wait_plan(p->inner2);
}

// allocate and upload the tables (called after every argument check passed)
int finish_plan(fft_plan* p, const std::vector<std::vector<float2>*>& parts,
                const std::vector<const float2**>& slots, size_t scratch_bytes) {
  std::vector<float2> all;
  std::vector<size_t> offs;
  for (auto* v : parts) {
    while (all.size() % 32) all.push_back(make_float2(0.f, 0.f));  // 256 B alignment
    offs.push_back(all.size());
    all.insert(all.end(), v->begin(), v->end());
  }
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) return hip_err(e, "hipGetDevice");
  // Plan memory comes from the device's stream-ordered pool (allocated on
  // the null stream, then synchronised, so every stream may use it) and is
  // returned with hipFreeAsync: hipFree synchronises the whole device, which
  // would make fft_plan_destroy wait for unrelated streams.
  e = hipMallocAsync((void**)&p->tables, all.size() * sizeof(float2), nullptr);
  if (e != hipSuccess) return hip_err(e, "hipMallocAsync(twiddle tables)");
  e = hipMemcpy(p->tables, all.data(), all.size() * sizeof(float2), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_err(e, "hipMemcpy(twiddle tables)");
  for (size_t i = 0; i < slots.size(); ++i) *slots[i] = p->tables + offs[i];
  if (scratch_bytes) {
    e = hipMallocAsync((void**)&p->scratch, scratch_bytes, nullptr);
    if (e != hipSuccess) return hip_err(e, "hipMallocAsync(scratch)");
    p->scratch_bytes = scratch_bytes;
  }
  e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) return hip_err(e, "hipStreamSynchronize");
  e = hipEventCreateWithFlags(&p->done, hipEventDisableTiming);
  if (e != hipSuccess) return hip_err(e, "hipEventCreateWithFlags");
  return FFT_OK;
}

// direct kinds: the table e^{-2 pi i u/n} = (cos, -sin)(2 pi u/n), u = 0..n/2
fft_plan* create_direct(int64_t n, int64_t batch, int kind, int sign) {
  if (n < 2 || n > kMaxDirectLength)
    return set_err(FFT_ENOTSUP, "direct kinds need 2 <= n <= 16384"), nullptr;
  fft_plan* p = new (std::nothrow) fft_plan();
  if (!p) return set_err(FFT_ENOMEM, "host allocation failed"), nullptr;
  p->n = n;
  p->nx = n;
  p->batch = batch;
  p->kind = kind;
  p->sign = sign;
  p->mmax = (n - 1) / 2;
  std::vector<float2> trig;
  for (int64_t u = 0; u <= n / 2; ++u) trig.push_back(root(u, n));
  if (finish_plan(p, {&trig}, {&p->trig}, 0) != FFT_OK) {
    free_plan(p);
    return nullptr;
  }
  ok();
  return p;
}

// Radices of the mixed-radix schedule: the fewest factors of n from `set`
// (descending) that are all >= rlo (so that no stage has more than n/rlo
// butterflies); among those the most even ones (smallest ratio of the
// largest to the smallest radix: with one butterfly per thread, a stage of
// large radix leaves most threads idle), then the larger smallest radix.
// Empty when there is none (n has a prime factor the set lacks, or needs
// smaller radices).  With the composite radices 10, 12, 14, 15 and 16, 1000 is
// 10 x 10 x 10: three stages and two LDS round trips instead of 8 x 5 x 5 x 5.
// The fixed-order schedule with radices up to 8: 8s (with 4 x 4 in place of
// 8 x 2), the leftover 4 or 2, then 7s, 5s and 3s; empty when n has another
// prime factor.
std::vector<int> mixed_radices_fixed(int64_t n) {
  std::vector<int> r;
  int a = 0;
  while (n % 2 == 0) n /= 2, ++a;
  if (a % 3 == 1 && a >= 4) {
    for (int i = 0; i < a / 3 - 1; ++i) r.push_back(8);
    r.push_back(4);
    r.push_back(4);
  } else {
    for (int i = 0; i < a / 3; ++i) r.push_back(8);
    if (a % 3 == 2) r.push_back(4);
    if (a % 3 == 1) r.push_back(2);
  }
  for (int p : {7, 5, 3})
    while (n % p == 0) n /= p, r.push_back(p);
  if (n != 1) r.clear();
  return r;
}

std::vector<int> mixed_radices(int64_t n, const std::vector<int>& set, int rlo) {
  std::vector<int> best, cur;
  std::function<void(int64_t, size_t)> dfs = [&](int64_t m, size_t from) {
    if (m == 1) {
      // cur and best are descending: front() is the largest radix, back() the smallest
      const bool better =
          best.empty() || cur.size() < best.size() ||
          (cur.size() == best.size() &&
           (cur.front() * best.back() < best.front() * cur.back() ||
            (cur.front() * best.back() == best.front() * cur.back() && cur.back() > best.back())));
      if (better) best = cur;
      return;
    }
    if (!best.empty() && cur.size() >= best.size()) return;
    for (size_t i = from; i < set.size(); ++i) {
      if (set[i] < rlo) break;
      if (m % set[i] != 0) continue;
      cur.push_back(set[i]);
      dfs(m / set[i], i);
      cur.pop_back();
    }
  };
  dfs(n, 0);
  return best;
}

// C2C of a length with no prime factor above 13, not a power of two, <= kMaxMixedLength
fft_plan* create_mixed(int64_t n, int64_t batch, int sign, const std::vector<int>& rad, int kb) {
  fft_plan* p = new (std::nothrow) fft_plan();
  if (!p) return set_err(FFT_ENOMEM, "host allocation failed"), nullptr;
  p->n = n;
  p->nx = n;
  p->batch = batch;
  p->kind = FFT_C2C;
  p->sign = sign;
  p->mixed = true;
  MixedArgs& a = p->mx;
  a.rows = batch;
  a.n = (int)n;
  a.nstages = (int)rad.size();
  std::vector<float2> tw, sh, ish;
  int64_t ns = 1, maxm = 0;
  for (int st = 0; st < a.nstages; ++st) {
    const int R = rad[st];
    a.radix[st] = R;
    a.ns[st] = (int)ns;
    a.m[st] = (int)(n / R);
    a.ns_magic[st] = ns == 1 ? 0u : (uint32_t)(((uint64_t(1) << 32) + (uint64_t)ns - 1) / (uint64_t)ns);
    a.twoff[st] = (int)tw.size();
    if (st > 0)
      for (int r = 1; r < R; ++r)
        for (int64_t j = 0; j < ns; ++j) tw.push_back(root((int64_t)r * j, ns * R));
    maxm = std::max<int64_t>(maxm, n / R);
    ns *= R;
  }
  if (tw.empty()) tw.push_back(make_float2(1.f, 0.f));
  a.kb = kb;
  // LDS padding: one element every 32 when the first stage is radix 16 (its
  // writes are 16 elements apart), none otherwise (the stage reads are runs
  // that a pad splits).  Measured on MI355X against padding every schedule:
  // first radix 16 (1280, 1536, 1792, 2560, 3072, 3584) 3-8 % faster with the
  // pad; first radix 8, 10, 12, 14 (48 ... 7168) equal or up to 7.6 % faster
  // without it (6400 383.7 -> 357.7 us, 7168 379.9 -> 351.2 us per 512 MiB).
  a.pad = rad[0] == 16 && kb == 1 ? 1 : 0;
  a.tpl = (int)((maxm + a.kb - 1) / a.kb);
  // 256 threads per workgroup where a line has fewer.  Filling the last
  // wavefront with more lines per workgroup (n = 1000: 7 lines, 700 of 704
  // lanes busy, against 200 of 256) was measured slower on MI355X: 1000 1.06x,
  // 2000 1.32x, 360 1.40x the time, from fewer workgroups per CU.
  a.lines = a.tpl >= 256 ? 1 : 256 / a.tpl;
  // shift factors of odd n, e^{-sign 2 pi i j h/n} and e^{+sign ...}, h =
  // floor(n/2) ("The 1D fftshift in CUDA by chessboard multiplication", odd
  // case); for even n the kernel flips the signs of odd j exactly instead
  const int64_t h = n / 2;
  if (n % 2 == 0) sh.push_back(make_float2(1.f, 0.f)), ish.push_back(make_float2(1.f, 0.f));
  for (int64_t j = 0; n % 2 == 1 && j < n; ++j) {
    const float2 w = root((j * h) % n, n);  // e^{-2 pi i jh/n}
    const float2 wc = make_float2(w.x, -w.y);
    sh.push_back(sign < 0 ? wc : w);
    ish.push_back(sign < 0 ? w : wc);
  }
  if (finish_plan(p, {&tw, &sh, &ish}, {&a.tw, &p->mx_shift, &p->mx_ishift}, 0) != FFT_OK) {
    free_plan(p);
    return nullptr;
  }
  ok();
  return p;
}

// A schedule of N with one butterfly per thread (radices up to 16) into a,
// its stage twiddles appended to tw; lines per workgroup and padding as for
// the mixed-radix plans.  Used by the transforms whose N-point stages run on
// a line in LDS (Rader, Bluestein on a mixed-radix length).
void fill_schedule(MixedArgs& a, int64_t N, const std::vector<int>& rad, std::vector<float2>& tw, int kb = 1) {
  a.n = (int)N;
  a.nstages = (int)rad.size();
  int64_t ns = 1, maxm = 0;
  for (int st = 0; st < a.nstages; ++st) {
    const int R = rad[st];
    a.radix[st] = R;
    a.ns[st] = (int)ns;
    a.m[st] = (int)(N / R);
    a.ns_magic[st] = ns == 1 ? 0u : (uint32_t)(((uint64_t(1) << 32) + (uint64_t)ns - 1) / (uint64_t)ns);
    a.twoff[st] = (int)tw.size();
    if (st > 0)
      for (int r = 1; r < R; ++r)
        for (int64_t j = 0; j < ns; ++j) tw.push_back(root((int64_t)r * j, ns * R));
    maxm = std::max<int64_t>(maxm, N / R);
    ns *= R;
  }
  if (tw.empty()) tw.push_back(make_float2(1.f, 0.f));
  a.kb = kb;
  a.pad = rad[0] == 16 && kb == 1 ? 1 : 0;
  a.tpl = (int)((maxm + kb - 1) / kb);
  a.lines = a.tpl >= 256 ? 1 : 256 / a.tpl;
}

// C2C of a prime length p by Rader's algorithm: a cyclic convolution of
// length N = p - 1 on the mixed-radix schedule rad of N (kb butterflies per
// thread, radices up to 16).  Tables: the stage twiddles of N, conv (the f64
// transform of b_m = e^{sign 2 pi i g^m/p}, divided by N), the index pairs
// of each j, and the shift ramps.
fft_plan* create_rader(int64_t p_len, int64_t batch, int sign, const std::vector<int>& rad, int kb = 1) {
  fft_plan* p = new (std::nothrow) fft_plan();
  if (!p) return set_err(FFT_ENOMEM, "host allocation failed"), nullptr;
  const int64_t n = p_len, N = n - 1;
  p->n = n;
  p->nx = n;
  p->batch = batch;
  p->kind = FFT_C2C;
  p->sign = sign;
  p->rader = true;
  MixedArgs& a = p->mx;
  a.rows = batch;
  std::vector<float2> tw, conv, perm, sh, ish;
  fill_schedule(a, N, rad, tw, kb);
  // generator powers and discrete logarithms
  const int64_t g = primitive_root(n);
  std::vector<int64_t> ind(n, 0);
  for (int64_t q = 0, gq = 1; q < N; ++q, gq = gq * g % n) ind[gq] = q;
  std::vector<std::complex<double>> b(N);
  for (int64_t m = 0, gm = 1; m < N; ++m, gm = gm * g % n) {
    const double ang = (double)sign * kTwoPi * (double)gm / (double)n;
    b[m] = std::complex<double>(std::cos(ang), std::sin(ang));
  }
  host_dft_f64(b);
  for (int64_t k = 0; k < N; ++k)
    conv.push_back(make_float2((float)(b[k].real() / (double)N), (float)(b[k].imag() / (double)N)));
  for (int64_t j = 0; j < n; ++j) {
    const int32_t in_pos = j == 0 ? 0 : (int32_t)((N - ind[j]) % N);
    const int32_t out_pos = j == 0 ? 0 : (int32_t)ind[j];
    float2 v;
    std::memcpy(&v.x, &in_pos, sizeof(float));
    std::memcpy(&v.y, &out_pos, sizeof(float));
    perm.push_back(v);
  }
  // shift factors of an odd length (as for the mixed-radix plans)
  const int64_t h = n / 2;
  for (int64_t j = 0; j < n; ++j) {
    const float2 w = root((j * h) % n, n);
    const float2 wc = make_float2(w.x, -w.y);
    sh.push_back(sign < 0 ? wc : w);
    ish.push_back(sign < 0 ? w : wc);
  }
  if (finish_plan(p, {&tw, &conv, &perm, &sh, &ish}, {&a.tw, &p->rd_conv, &p->rd_perm, &p->mx_shift, &p->mx_ishift},
                  0) != FFT_OK) {
    free_plan(p);
    return nullptr;
  }
  ok();
  return p;
}

// C2C of a length that is not a power of two, 2 <= n <= kMaxBluesteinLengthLarge.
// The transforms of length m >= 2n - 1 run inside one kernel per row batch
// while m <= 2 * kMaxBluesteinLength; above, in three passes over batch x m values
// through two plan-owned scratch buffers: the forward transform's column
// pass with the chirp applied on load, one row pass for the forward row
// factor, the product with bhat and the inverse row factor, and the inverse
// column pass with the chirp applied on store.
fft_plan* create_bluestein(int64_t n, int64_t batch, int sign) {
  fft_plan* p = new (std::nothrow) fft_plan();
  if (!p) return set_err(FFT_ENOMEM, "host allocation failed"), nullptr;
  p->n = n;
  p->nx = n;
  p->batch = batch;
  p->kind = FFT_C2C;
  p->sign = sign;
  p->bluestein = true;
  int64_t m = 1;
  while (m < 2 * n - 1) m <<= 1;
  // A convolution length with a mixed-radix schedule where it is much
  // shorter than the power of two (n just above a power of two: 1034 can use
  // 2080 = 16 x 13 x 10 instead of 4096).  Among the lengths c >= 2n - 1 with
  // 1.3 c < m, the one with the smallest c x stages.  Measured on MI355X per
  // 512 MiB: 1034 973 -> 908 us, 1049 966 -> 863 us, 2053 1325 -> 1139 us,
  // 2111 1298 -> 1044 us; with the short lines read and written through LDS
  // also below 4096: 34 (70 = 10 x 7) 797 -> 473 us, 47 (96) 663 -> 462, 83
  // (168) 686 -> 464, 167 728 -> 696, 263 (525) 871 -> 790.
  std::vector<int> msched;
  if (m >= 64) {
    static const std::vector<int> wide = {16, 15, 14, 13, 12, 11, 10, 8, 7, 6, 5, 4, 3, 2};
    int64_t best_cost = INT64_MAX, best_c = 0;
    for (int64_t c = 2 * n - 1; c <= kMaxChirpMixedLength && 13 * c < 10 * m && 2 * c < best_cost; ++c) {
      const std::vector<int> w = mixed_radices(c, wide, (int)((c + 1023) / 1024));
      if (w.empty() || (int)w.size() > kMixedMaxStages) continue;
      if (c * (int64_t)w.size() < best_cost) best_cost = c * (int64_t)w.size(), best_c = c, msched = w;
    }
    if (best_c) m = best_c, p->bmixed = true;
  }
  p->bm = (int)m;
  std::vector<float2> ta, tb, thi, tlo, pre, pres, prei, bh, bht;
  size_t scratch = 0;
  if (p->bmixed) {
    p->mx.rows = batch;
    fill_schedule(p->mx, m, msched, ta);
  } else if (m <= 2 * (int64_t)kMaxBluesteinLength) {  // one kernel (k_bluestein.hip)
    append_stage_table((int)m, m > kMaxSinglePass ? kSplitValues : rows_values((int)m), ta);
  } else {
    const int L = ilog2c(m);
    p->fourstep = true;
    p->n1 = 1 << (L / 2);
    p->n2 = 1 << (L - L / 2);
    p->bits = L - L / 2;
    append_stage_table(p->n1, tposed_values(p->n1), ta);
    append_stage_table(p->n2, cols_values(p->n2), tb);
    for (int64_t hh = 0; hh < (m >> p->bits); ++hh) thi.push_back(root(hh << p->bits, m));
    for (int64_t l = 0; l < (int64_t(1) << p->bits); ++l) tlo.push_back(root(l, m));
    scratch = 2 * (size_t)(m * batch) * sizeof(float2);
  }
  // c_j = e^{sign pi i j^2/n}; with the shift, times e^{-sign 2 pi i j h/n},
  // h = floor(n/2), which moves bin 0 to index h ("The 1D fftshift in CUDA by
  // chessboard multiplication": (-1)^j for even n, a complex ramp for odd n);
  // with the inverse shift, times e^{+sign 2 pi i j h/n}, which moves index h
  // to 0 (the same for even n)
  const int64_t h = n / 2;
  for (int64_t j = 0; j < n; ++j) {
    pre.push_back(chirp(j * j, n, sign));
    pres.push_back(chirp(j * j - 2 * j * h, n, sign));
    prei.push_back(chirp(j * j + 2 * j * h, n, sign));
  }
  // b = conj(c) wrapped around to length m, transformed in f64, divided by m
  std::vector<std::complex<double>> b((size_t)m, 0.0);
  for (int64_t j = 0; j < n; ++j) {
    const int64_t r = (j * j) % (2 * n);
    const double a = kTwoPi * 0.5 * (double)r / (double)n;
    const std::complex<double> cb(std::cos(a), -sign * std::sin(a));
    b[(size_t)j] = cb;
    if (j > 0) b[(size_t)(m - j)] = cb;
  }
  if (p->bmixed)
    host_dft_f64(b);
  else
    host_fft_f64(b);
  for (int64_t k = 0; k < m; ++k) {
    const std::complex<double> v = b[(size_t)k] / (double)m;
    bh.push_back(make_float2((float)v.real(), (float)v.imag()));
  }
  std::vector<std::vector<float2>*> parts = {&ta, &pre, &pres, &prei, &bh};
  std::vector<const float2**> slots = {p->bmixed ? &p->mx.tw : &p->tw_a, &p->chirp, &p->chirp_shift, &p->chirp_ishift,
                                       &p->bhat};
  if (p->fourstep) {
    // the row pass between the transforms reads bhat row by row: k2*n1 + k1
    for (int64_t k2 = 0; k2 < p->n2; ++k2)
      for (int64_t k1 = 0; k1 < p->n1; ++k1) bht.push_back(bh[(size_t)(k2 + p->n2 * k1)]);
    parts.insert(parts.end(), {&tb, &thi, &tlo, &bht});
    slots.insert(slots.end(), {&p->tw_b, &p->thi, &p->tlo, &p->bhat_t});
  }
  if (finish_plan(p, parts, slots, scratch) != FFT_OK) {
    free_plan(p);
    return nullptr;
  }
  ok();
  return p;
}

// any-length C2C plan: mixed radix when possible, then Rader for primes,
// else the chirp transform
// The one-kernel mixed-radix schedule of n <= kMaxMixedLength (kb: butterflies
// per thread), or an empty list.  In order:
//  1. radices up to 16, one butterfly per thread (1000: 10 10 10, three
//     stages).  Measured against the fixed order of step 3 on MI355X with
//     each stage compiled for its radix: better or equal for 1000, 2000,
//     2500 (253 against 330 us per 512 MiB), 3000, 3500, 4500, 6000, 8000,
//     worse for 4000 and 5000 (325 against 291, 289 against 280 us);
//  2. above 8192 points, radices up to 16 with two butterflies per thread
//     (one would need every radix >= n/1024).  Per 512 MiB against the chirp
//     transform: 10000 1331 -> 313 us, 9000 1440 -> 408, 12000 1133 -> 401,
//     16000 954 -> 416; against the p * 2^k kernel it replaced: 9216 444 ->
//     414, 10240 445 -> 429, 12288 404 -> 399, 12800 433 -> 394, 14336 399 ->
//     370, 15360 392 -> 372;
//  3. radices up to 8 in a fixed order, two butterflies per thread;
//  4. the fewest radices up to 8, two butterflies per thread (7776: 6^5).
std::vector<int> one_kernel_schedule(int64_t n, int* kb) {
  static const std::vector<int> wide = {16, 15, 14, 13, 12, 11, 10, 8, 7, 6, 5, 4, 3, 2};
  static const std::vector<int> narrow = {8, 7, 6, 5, 4, 3, 2};
  if (n < 2 || n > kMaxMixedLength) return {};
  std::vector<int> w = mixed_radices(n, wide, (int)((n + 1023) / 1024));
  if (!w.empty() && (int)w.size() <= kMixedMaxStages) return *kb = 1, w;
  const int rlo2 = (int)((n + 2 * 1024 - 1) / (2 * 1024));
  if (n > 8192) {
    w = mixed_radices(n, wide, rlo2);
    if (!w.empty() && (int)w.size() <= kMixedMaxStages) return *kb = kMixedButterflies, w;
  }
  for (const std::vector<int>& r : {mixed_radices_fixed(n), mixed_radices(n, narrow, rlo2)}) {
    if (r.empty() || (int)r.size() > kMixedMaxStages) continue;
    if (n / *std::min_element(r.begin(), r.end()) <= 1024 * kMixedButterflies) return *kb = kMixedButterflies, r;
  }
  return {};
}

bool smooth13(int64_t n) {
  for (int p : {2, 3, 5, 7, 11, 13})
    while (n % p == 0) n /= p;
  return n == 1;
}

// C2C of a length with no prime factor above 13 and no one-kernel schedule
// (above 16384 points, and a few below: 15625 = 5^6, 6561 = 3^8), as a
// four-step split n = n1 * n2 (the decomposition the ctsai page names for
// transforms that do not fit on chip, with mixed-radix factors): n2 <= 1024
// (16 columns of a tile fit the LDS) with the one-butterfly schedule, n2
// closest to sqrt(n).  Two passes where n1 has a schedule for row tiles of
// at least 8 rows in LDS (n1 up to about 2540): the column tiles with the
// twiddle into the scratch, then row tiles stored transposed; else three
// (n1 a power of two up to 16384 or a one-kernel length): the row plan of
// n1 in place on the scratch, then the transpose.  Returns nullptr with
// *split false when no split exists.
bool tile_schedule(int64_t n, std::vector<int>* w, int* kb) {
  *w = one_kernel_schedule(n, kb);
  if (w->empty()) return false;
  const int rmax = *std::max_element(w->begin(), w->end());
  if (rmax > 8 && *kb != 1) return false;  // no tile kernel of this shape
  const bool pad = (*w)[0] == 16 && *kb == 1;
  const int64_t pitch = (pad ? n + n / 32 : n) + 1;
  return 8 * pitch * (int64_t)sizeof(float2) <= kLdsBudgetBytes;
}

fft_plan* create_fourstep_any(int64_t n, int64_t batch, int sign, bool* split) {
  *split = false;
  if (n < 4 || n > kMaxBluesteinLengthLarge || !smooth13(n)) return nullptr;
  int64_t best = 0;
  bool best2 = false;
  double bestd = 1e300;
  std::vector<int> w2best, w1best;
  int kb1best = 1;
  for (int64_t n2 = 2; n2 <= 1024 && n2 < n; ++n2) {
    if (n % n2) continue;
    const int64_t n1 = n / n2;
    int kb1 = 0, kb2 = 0;
    std::vector<int> w1;
    const bool two = n1 >= 2 && n1 <= kMaxMixedLength && tile_schedule(n1, &w1, &kb1);
    if (!two && (n1 < 2 || n1 > kMaxMixedLength || (!is_pow2(n1) && one_kernel_schedule(n1, &kb1).empty())))
      continue;
    const std::vector<int> w2 = one_kernel_schedule(n2, &kb2);
    if (w2.empty() || kb2 != 1) continue;
    const double d = std::fabs(std::log((double)n2) - 0.5 * std::log((double)n));
    if ((two && !best2) || (two == best2 && d < bestd))
      bestd = d, best = n2, best2 = two, w2best = w2, w1best = w1, kb1best = kb1;
  }
  if (!best) return nullptr;
  *split = true;
  const int64_t n2 = best, n1 = n / n2;
  fft_plan* rows = best2 ? create_mixed(n1, 1, sign, w1best, kb1best) : fft_plan_create(n1, batch * n2, FFT_C2C, sign);
  if (!rows) return nullptr;
  fft_plan* cols = create_mixed(n2, 1, sign, w2best, 1);
  if (!cols) {
    free_plan(rows);
    return nullptr;
  }
  fft_plan* p = new (std::nothrow) fft_plan();
  if (!p) {
    free_plan(rows);
    free_plan(cols);
    return set_err(FFT_ENOMEM, "host allocation failed"), nullptr;
  }
  p->n = n;
  p->nx = n;
  p->batch = batch;
  p->kind = FFT_C2C;
  p->sign = sign;
  p->fsany = true;
  p->fs2 = best2;
  p->n1 = (int)n1;
  p->n2 = (int)n2;
  p->bits = (ilog2c(n) + 1) / 2;
  p->inner = rows;
  p->inner2 = cols;
  std::vector<float2> thi, tlo;
  for (int64_t h = 0; h <= ((n - 1) >> p->bits); ++h) thi.push_back(root(h << p->bits, n));
  for (int64_t l = 0; l < (int64_t(1) << p->bits); ++l) tlo.push_back(root(l, n));
  if (finish_plan(p, {&thi, &tlo}, {&p->thi, &p->tlo}, (size_t)(n * batch) * sizeof(float2)) != FFT_OK) {
    free_plan(p);
    return nullptr;
  }
  ok();
  return p;
}

fft_plan* create_c2c_any(int64_t n, int64_t batch, int sign) {
  // The mixed-radix kernel up to 16384 points (one_kernel_schedule), else
  // the mixed-radix four-step, else Rader (primes), else the chirp
  // transform.  (An earlier p * 2^k kernel for n = p * 2^k, p in {3, 5, 7, 9,
  // 15, 25}, lost to mixed radix on every length it took: 3072 216 against
  // 310 us, 6144 266 against 312, 15360 372 against 392 per 512 MiB.)
  int kb = 0;
  const std::vector<int> w = one_kernel_schedule(n, &kb);
  if (!w.empty()) return create_mixed(n, batch, sign, w, kb);
  bool split = false;
  fft_plan* q = create_fourstep_any(n, batch, sign, &split);
  if (split) return q;  // nullptr: its plans failed, the error is set
  // primes up to 16385 whose p - 1 has a schedule: Rader's convolution of
  // length p - 1 in one kernel (1009: two 1008-point transforms instead of
  // the chirp transform's two of 2048)
  if (n <= kMaxMixedLength + 1 && is_prime(n)) {
    static const std::vector<int> wide = {16, 15, 14, 13, 12, 11, 10, 8, 7, 6, 5, 4, 3, 2};
    const std::vector<int> wr = mixed_radices(n - 1, wide, (int)((n - 1 + 1023) / 1024));
    if (!wr.empty() && (int)wr.size() <= kMixedMaxStages) return create_rader(n, batch, sign, wr);
    if (n - 1 > 8192) {  // two butterflies per thread, as for the mixed-radix lengths above 8192
      const std::vector<int> wr2 = mixed_radices(n - 1, wide, (int)((n - 1 + 2047) / 2048));
      if (!wr2.empty() && (int)wr2.size() <= kMixedMaxStages)
        return create_rader(n, batch, sign, wr2, kMixedButterflies);
    }
  }
  return create_bluestein(n, batch, sign);
}

// R2C/C2R of a length that is not a power of two (3 <= n <= kMaxBluesteinLengthLarge),
// or of a power of two above the one-kernel real rows (n/2 on the four-step path)
fft_plan* create_real_any(int64_t n, int64_t batch, int kind, int sign) {
  const bool even = n % 2 == 0;
  const int64_t len = even ? n / 2 : n;
  fft_plan* inner = is_pow2(len) ? fft_plan_create(len, batch, FFT_C2C, sign) : create_c2c_any(len, batch, sign);
  if (!inner) return nullptr;
  fft_plan* p = new (std::nothrow) fft_plan();
  if (!p) {
    free_plan(inner);
    return set_err(FFT_ENOMEM, "host allocation failed"), nullptr;
  }
  p->n = n;
  p->nx = n;
  p->batch = batch;
  p->kind = kind;
  p->sign = sign;
  p->mmax = n / 2;
  p->real_any = true;
  p->inner = inner;
  std::vector<float2> trt;
  for (int64_t k = 0; k <= n / 2; ++k) trt.push_back(root(k, n));
  const size_t scratch = (size_t)(batch * len) * sizeof(float2) * (even ? 1 : 2);
  if (finish_plan(p, {&trt}, {&p->rt}, scratch) != FFT_OK) {
    free_plan(p);
    return nullptr;
  }
  ok();
  return p;
}

}  // namespace

extern "C" {

fft_plan* fft_plan_create(int64_t n, int64_t batch, int kind, int sign) {
  if (n < 1) return set_err(FFT_EINVAL, "n must be >= 1"), nullptr;
  if (batch < 1) return set_err(FFT_EINVAL, "batch must be >= 1"), nullptr;
  if (check_kind_sign(kind, sign) != FFT_OK) return nullptr;
  if (check_total(n, batch, 1) != FFT_OK) return nullptr;
  if (is_direct(kind)) return create_direct(n, batch, kind, sign);
  if (kind == FFT_C2C && n > 1 && !is_pow2(n)) {
    if (n > kMaxBluesteinLengthLarge)
      return set_err(FFT_ENOTSUP, "C2C lengths that are not powers of two must be <= 2^22"), nullptr;
    // mixed radix when every prime factor is at most 13 and every stage has
    // at most 1024 butterflies per thread slot, Rader for primes, else the
    // chirp transform
    return create_c2c_any(n, batch, sign);
  }
  if (kind != FFT_C2C && n > 2 && !is_pow2(n)) {
    if (n > kMaxBluesteinLengthLarge)
      return set_err(FFT_ENOTSUP, "R2C/C2R lengths that are not powers of two must be <= 2^22"), nullptr;
    return create_real_any(n, batch, kind, sign);
  }
  if (!is_pow2(n)) return set_err(FFT_ENOTSUP, "n out of range"), nullptr;
  const int64_t max_len = int64_t(1) << (kind == FFT_C2C ? kFourStepMaxLog : kFourStepMaxLog + 1);
  const int64_t min_len = kind == FFT_C2C ? 2 : 4;
  if (n < min_len || n > max_len)
    return set_err(FFT_ENOTSUP, "n out of range: C2C needs 2 <= n <= 2^28, R2C/C2R 4 <= n <= 2^29"),
           nullptr;
  // real rows above one kernel's reach: the four-step transform of n/2
  // complex values, then the Hermitian unpack (pack first for C2R)
  if (kind != FFT_C2C && n > 2 * (int64_t)kMaxSinglePass) return create_real_any(n, batch, kind, sign);

  fft_plan* p = new (std::nothrow) fft_plan();
  if (!p) return set_err(FFT_ENOMEM, "host allocation failed"), nullptr;
  p->dims = 1;
  p->n = n;
  p->nx = n;
  p->batch = batch;
  p->kind = kind;
  p->sign = sign;
  p->mmax = n / 2;

  std::vector<float2> ta, tb, trt, thi, tlo;
  std::vector<std::vector<float2>*> parts;
  std::vector<const float2**> slots;
  size_t scratch = 0;
  if (kind == FFT_C2C && n <= kMaxSinglePass) {
    append_stage_table((int)n, rows_values((int)n), ta);
    parts = {&ta};
    slots = {&p->tw_a};
  } else if (kind == FFT_C2C) {
    const int L = ilog2c(n);
    p->fourstep = true;
    p->n1 = 1 << (L / 2);
    p->n2 = 1 << (L - L / 2);
    p->bits = L - L / 2;
    append_stage_table(p->n1, tposed_values(p->n1), ta);
    append_stage_table(p->n2, cols_values(p->n2), tb);
    for (int64_t h = 0; h < (n >> p->bits); ++h) thi.push_back(root(h << p->bits, n));
    for (int64_t l = 0; l < (int64_t(1) << p->bits); ++l) tlo.push_back(root(l, n));
    parts = {&ta, &tb, &thi, &tlo};
    slots = {&p->tw_a, &p->tw_b, &p->thi, &p->tlo};
    scratch = (size_t)(n * batch) * sizeof(float2);
  } else {
    append_stage_table((int)(n / 2), real_values((int)(n / 2)), ta);
    for (int64_t k = 0; k <= n / 2; ++k) trt.push_back(root(k, n));
    parts = {&ta, &trt};
    slots = {&p->tw_a, &p->rt};
    if (n <= kMaxSinglePass) {  // for FFT_OPT_REAL_PAIRS
      append_stage_table((int)n, real_values((int)n), tb);
      parts.push_back(&tb);
      slots.push_back(&p->tw_full);
    }
  }
  if (finish_plan(p, parts, slots, scratch) != FFT_OK) {
    free_plan(p);
    return nullptr;
  }
  ok();
  return p;
}

fft_plan* fft_plan_create_2d(int64_t ny, int64_t nx, int64_t batch, int kind, int sign) {
  if (ny < 1 || nx < 1) return set_err(FFT_EINVAL, "ny and nx must be >= 1"), nullptr;
  if (batch < 1) return set_err(FFT_EINVAL, "batch must be >= 1"), nullptr;
  if (check_kind_sign(kind, sign) != FFT_OK) return nullptr;
  if (kind != FFT_C2C) return set_err(FFT_ENOTSUP, "2D plans support FFT_C2C only"), nullptr;
  if (!is_pow2(ny) || !is_pow2(nx)) {
    // rows, transpose, rows of the transposed image, transpose back
    if (ny < 2 || nx < 2 || ny > kMaxBluesteinLengthLarge || nx > kMaxBluesteinLengthLarge)
      return set_err(FFT_ENOTSUP, "2D sizes that are not powers of two must lie in [2, 2^22]"), nullptr;
    if (check_total(ny, nx, batch) != FFT_OK) return nullptr;
    if (batch > 65535)
      return set_err(FFT_ENOTSUP, "2D plans with a size that is not a power of two take at most 65535 images"),
             nullptr;
    // The column pass runs in place on the columns (two HBM passes with the
    // rows) when ny is a power of two whose column tile holds at least 8
    // columns (64 B runs), or has a mixed-radix schedule whose tile does;
    // else the image is transposed, transformed as rows and transposed back.
    fft_plan* rows = fft_plan_create(nx, batch * ny, FFT_C2C, sign);
    if (!rows) return nullptr;
    int cols2d = 0;
    fft_plan* cols = nullptr;
    if (is_pow2(ny) && ny <= kMaxSinglePass && tile_lines((int)ny, false) >= 8) {
      cols2d = 1;
    } else {
      cols = fft_plan_create(ny, is_pow2(ny) ? 1 : batch * nx, FFT_C2C, sign);
      if (!cols) {
        free_plan(rows);
        return nullptr;
      }
      if (cols->mixed && mixed_cols_tile(cols->mx) >= 8 && ny * nx <= (int64_t(1) << 29)) cols2d = 2;
      if (cols2d == 0 && is_pow2(ny)) {  // the transposed rows need a plan of the full batch
        free_plan(cols);
        cols = fft_plan_create(ny, batch * nx, FFT_C2C, sign);
        if (!cols) {
          free_plan(rows);
          return nullptr;
        }
      }
    }
    fft_plan* p = new (std::nothrow) fft_plan();
    if (!p) {
      free_plan(rows);
      free_plan(cols);
      return set_err(FFT_ENOMEM, "host allocation failed"), nullptr;
    }
    p->dims = 2;
    p->ny = ny;
    p->nx = nx;
    p->n = ny * nx;
    p->batch = batch;
    p->kind = kind;
    p->sign = sign;
    p->any2d = true;
    p->cols2d = cols2d;
    p->inner = rows;
    p->inner2 = cols;
    std::vector<float2> tcols;
    if (cols2d == 1)
      append_stage_table((int)ny, cols_values((int)ny), tcols);
    else
      tcols.push_back(make_float2(0.f, 0.f));
    const size_t scratch = cols2d ? 0 : (size_t)(ny * nx * batch) * sizeof(float2);
    if (finish_plan(p, {&tcols}, {&p->tw_b}, scratch) != FFT_OK) {
      free_plan(p);
      return nullptr;
    }
    ok();
    return p;
  }
  if (ny < 2 || nx < 2 || ny > kMaxSinglePass || nx > kMaxSinglePass)
    return set_err(FFT_ENOTSUP, "2D sizes must lie in [2, 16384]"), nullptr;
  if (check_total(ny, nx, batch) != FFT_OK) return nullptr;
  if (ny >= kTallRows && batch > 65535)
    return set_err(FFT_ENOTSUP, "2D plans with ny >= 8192 take at most 65535 images"), nullptr;

  fft_plan* p = new (std::nothrow) fft_plan();
  if (!p) return set_err(FFT_ENOMEM, "host allocation failed"), nullptr;
  p->dims = 2;
  p->ny = ny;
  p->nx = nx;
  p->n = ny * nx;
  p->batch = batch;
  p->kind = kind;
  p->sign = sign;
  std::vector<float2> ta, tb, tca, tcb, wt;
  append_stage_table((int)nx, rows_values((int)nx), ta);
  int rc;
  // Images of 8192 rows and more, and the 4096-row images the two-pass form
  // takes (faster than rows + the 4096-point column pass, whose tiles hold
  // only 8 columns), go through a scratch; the others transform in place.
  if (ny >= kTallRows || fold_supported(ny, nx)) {
    p->tall = true;
    p->fold = fold_supported(ny, nx);
    if (p->fold) {
      const int na = fold_na(ny, nx), nb = (int)(ny / na);
      append_stage_table((int)nx, fold_row_values((int)nx, na), tca);
      append_stage_table(nb, fold_col_values(nb, fold_c(nb)), tcb);
    } else {
      const int nb = (int)(ny / kTallSplit);
      append_stage_table(nb, colstage_values(nb), tca);
      append_stage_table(kTallSplit, colstage_values(kTallSplit), tcb);
    }
    for (int64_t e = 0; e < ny; ++e) wt.push_back(root(e, ny));
    const size_t scratch = (size_t)(p->fold ? fold_scratch_elems(ny, nx, batch) : ny * nx * batch);
    rc = finish_plan(p, {&ta, &tca, &tcb, &wt}, {&p->tw_a, &p->tw_ca, &p->tw_cb, &p->wt},
                     scratch * sizeof(float2));
  } else {
    append_stage_table((int)ny, cols_values((int)ny), tb);
    rc = finish_plan(p, {&ta, &tb}, {&p->tw_a, &p->tw_b}, 0);
  }
  if (rc != FFT_OK) {
    free_plan(p);
    return nullptr;
  }
  ok();
  return p;
}

int fft_plan_set(fft_plan* p, int option, int64_t value) {
  if (!p) return set_err(FFT_EINVAL, "plan is NULL");
  if (p->executed) return set_err(FFT_ESTATE, "options must be set before the first fft_exec");
  switch (option) {
    case FFT_OPT_SHIFT:
      if (value < 0 || value > 2) return set_err(FFT_EINVAL, "FFT_OPT_SHIFT takes 0, 1 or 2");
      if (p->kind != FFT_C2C) return set_err(FFT_EINVAL, "FFT_OPT_SHIFT applies to C2C plans only");
      if (value && !p->bluestein && !p->mixed && !p->rader && !p->any2d && !p->fsany &&
          ((p->nx & 1) || (p->dims == 2 && (p->ny & 1))))
        return set_err(FFT_EINVAL, "FFT_OPT_SHIFT needs even lengths");
      if (p->any2d) {  // the shift of each axis: in its row plan, or in the column pass
        if (fft_plan_set(p->inner, FFT_OPT_SHIFT, value) != FFT_OK) return g_err.code;
        if (p->inner2 && fft_plan_set(p->inner2, FFT_OPT_SHIFT, value) != FFT_OK) return g_err.code;
      }
      p->shift = (int)value;
      return ok();
    case FFT_OPT_MMAX:
      if (p->kind == FFT_C2C) return set_err(FFT_EINVAL, "FFT_OPT_MMAX applies to R2C/C2R plans only");
      if (is_direct(p->kind) && (value < 0 || 2 * value >= p->n))
        return set_err(FFT_EINVAL, "direct kinds need 0 <= mmax and 2 mmax < n");
      if (value < 0 || value > p->n / 2) return set_err(FFT_EINVAL, "mmax must satisfy 0 <= mmax <= n/2");
      p->mmax = value;
      return ok();
    case FFT_OPT_SPEC_LAYOUT:
      if (p->kind == FFT_C2C)
        return set_err(FFT_EINVAL, "FFT_OPT_SPEC_LAYOUT applies to R2C/C2R plans only");
      if (value != 0 && value != 1) return set_err(FFT_EINVAL, "FFT_OPT_SPEC_LAYOUT takes 0 or 1");
      p->spec_layout = (int)value;
      return ok();
    case FFT_OPT_REAL_PAIRS:
      if (p->kind == FFT_C2C) return set_err(FFT_EINVAL, "FFT_OPT_REAL_PAIRS applies to R2C/C2R plans only");
      if (value != 0 && value != 1) return set_err(FFT_EINVAL, "FFT_OPT_REAL_PAIRS takes 0 or 1");
      if (is_direct(p->kind)) return set_err(FFT_EINVAL, "FFT_OPT_REAL_PAIRS applies to R2C/C2R plans only");
      if (value && (p->batch & 1)) return set_err(FFT_EINVAL, "FFT_OPT_REAL_PAIRS needs an even batch");
      if (value && !p->tw_full) return set_err(FFT_ENOTSUP, "FFT_OPT_REAL_PAIRS supports n <= 16384");
      p->real_pairs = (int)value;
      return ok();
    default:
      return set_err(FFT_EINVAL, "unknown option");
  }
}

int fft_plan_get_sizes(const fft_plan* p, int64_t* in_bytes, int64_t* out_bytes) {
  if (!p) return set_err(FFT_EINVAL, "plan is NULL");
  const int64_t cplx = p->batch * p->n * 8;
  const int64_t real = p->batch * p->n * 4;
  const int64_t spec = p->batch * (p->mmax + 1) * 8;
  int64_t i = cplx, o = cplx;
  if (p->kind == FFT_R2C || p->kind == FFT_R2C_DIRECT) i = real, o = spec;
  if (p->kind == FFT_C2R || p->kind == FFT_C2R_DIRECT) i = spec, o = real;
  if (in_bytes) *in_bytes = i;
  if (out_bytes) *out_bytes = o;
  return ok();
}

}  // extern "C"

namespace {

int check_exec_args(const fft_plan* p, const void* in, const void* out) {
  if (!p) return set_err(FFT_EINVAL, "plan is NULL");
  if (!in || !out) return set_err(FFT_EINVAL, "in and out must be device pointers");
  if (((uintptr_t)in & 7) || ((uintptr_t)out & 7)) return set_err(FFT_EINVAL, "buffers must be 8-byte aligned");
  if (p->kind != FFT_C2C && in == out) return set_err(FFT_EINVAL, "R2C/C2R cannot run in place");
  return FFT_OK;
}

// The launch sequence of plan p on `stream` (device already current), with
// `sc` as the plan's scratch.  Inner plans run through fft_exec.
int run_plan(fft_plan* p, const void* in, void* out, fft_stream_t stream_, float2* sc) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  hipError_t e = hipSuccess;
  const float2* src = static_cast<const float2*>(in);
  float2* dst = static_cast<float2*>(out);
  if (p->any2d && p->cols2d) {
    // rows (with the shift along x), then the columns in place on out (with
    // the shift along y)
    int rc = fft_exec(p->inner, in, out, stream_);
    if (rc != FFT_OK) return rc;
    if (p->cols2d == 1) {
      const ColsArgs c{dst, dst, p->tw_b, p->ny, p->nx, p->batch, p->shift ? 1 : 0};
      e = launch_c2c_cols((int)p->ny, p->sign, c, stream);
    } else {
      MixedArgs a = p->inner2->mx;
      a.in = dst;
      a.out = dst;
      // even ny: the exact sign flip of odd rows for either shift; odd ny: the ramps
      const bool even = p->ny % 2 == 0;
      a.flip = even && p->shift ? 1 : 0;
      a.pre = even ? nullptr
                   : p->shift == 1 ? p->inner2->mx_shift : p->shift == 2 ? p->inner2->mx_ishift : nullptr;
      e = launch_mixed_cols(p->sign, a, MixedColsArgs{p->nx, p->batch}, stream);
    }
    if (e != hipSuccess) return hip_err(e, "kernel launch");
    return FFT_OK;
  }
  if (p->any2d) {
    int rc = fft_exec(p->inner, in, out, stream_);
    if (rc == FFT_OK) e = launch_transpose(dst, sc, p->ny, p->nx, p->batch, stream);
    if (rc == FFT_OK && e == hipSuccess) rc = fft_exec(p->inner2, sc, sc, stream_);
    if (rc == FFT_OK && e == hipSuccess) e = launch_transpose(sc, dst, p->nx, p->ny, p->batch, stream);
    if (rc != FFT_OK) return rc;
    if (e != hipSuccess) return hip_err(e, "kernel launch");
    return FFT_OK;
  }
  if (p->fsany) {
    // the n2-point columns (stride n1) times W_n^{j1 k2} into the scratch,
    // the n1-point rows in place there, then [n2][n1] -> [n1][n2] per row of
    // the batch, rotated by the shift (bin 0 to index n/2, or back)
    MixedArgs a = p->inner2->mx;
    a.in = src;
    a.out = sc;
    a.flip = 0;
    a.pre = nullptr;
    e = launch_mixed_cols(p->sign, a, MixedColsArgs{p->n1, p->batch, p->thi, p->tlo, p->bits, 0}, stream);
    const int64_t h = p->n / 2;
    const int64_t rot = p->shift == 1 ? h : p->shift == 2 ? (p->n - h) % p->n : 0;
    if (p->fs2) {  // row tiles of n1 stored transposed straight to out
      MixedArgs r = p->inner->mx;
      r.in = sc;
      r.out = dst;
      r.flip = 0;
      r.pre = nullptr;
      if (e == hipSuccess)
        e = launch_mixed_rows_t(p->sign, r, MixedColsArgs{p->n2, p->batch, nullptr, nullptr, 0, rot}, stream);
      if (e != hipSuccess) return hip_err(e, "kernel launch");
      return FFT_OK;
    }
    int rc = FFT_OK;
    if (e == hipSuccess) rc = fft_exec(p->inner, sc, sc, stream_);
    for (int64_t b0 = 0; b0 < p->batch && e == hipSuccess && rc == FFT_OK; b0 += 65535) {
      const int64_t nb = std::min<int64_t>(65535, p->batch - b0);
      e = launch_transpose(sc + b0 * p->n, dst + b0 * p->n, p->n2, p->n1, nb, stream, rot);
    }
    if (rc != FFT_OK) return rc;
    if (e != hipSuccess) return hip_err(e, "kernel launch");
    return FFT_OK;
  }
  if (p->real_any) {
    const bool even = p->n % 2 == 0;
    const int64_t len = even ? p->n / 2 : p->n;
    float2* s1 = sc;
    float2* s2 = sc + p->batch * len;
    RealAnyArgs ra{nullptr, nullptr, p->rt, p->batch, (int)p->n, (int)len, (int)p->mmax, p->spec_layout};
    int rc = FFT_OK;
    if (p->kind == FFT_R2C && even) {
      rc = fft_exec(p->inner, in, s1, stream_);  // x read as len complex values per row
      if (rc == FFT_OK) ra.in = s1, ra.out = out, e = launch_real_unpack(ra, stream);
    } else if (p->kind == FFT_R2C) {
      ra.in = in, ra.out = s1, e = launch_real_complexify(ra, stream);
      if (e == hipSuccess) rc = fft_exec(p->inner, s1, s2, stream_);
      if (e == hipSuccess && rc == FFT_OK) ra.in = s2, ra.out = out, e = launch_real_extract(ra, stream);
    } else if (even) {
      ra.in = in, ra.out = s1, e = launch_real_pack(ra, stream);
      if (e == hipSuccess) rc = fft_exec(p->inner, s1, out, stream_);  // x written as len complex values
    } else {
      ra.in = in, ra.out = s1, e = launch_real_hermitian(ra, stream);
      if (e == hipSuccess) rc = fft_exec(p->inner, s1, s2, stream_);
      if (e == hipSuccess && rc == FFT_OK) ra.in = s2, ra.out = out, e = launch_real_part(ra, stream);
    }
    if (rc != FFT_OK) return rc;
    if (e != hipSuccess) return hip_err(e, "kernel launch");
    return FFT_OK;
  }
  if (p->mixed) {
    MixedArgs a = p->mx;
    a.in = src;
    a.out = dst;
    // even n: both shifts are the exact sign flip (-1)^j; odd n: the ramps
    const bool even = p->n % 2 == 0;
    a.flip = even && p->shift ? 1 : 0;
    a.pre = even ? nullptr : p->shift == 1 ? p->mx_shift : p->shift == 2 ? p->mx_ishift : nullptr;
    e = launch_mixed(p->sign, a, stream);
  } else if (p->rader) {  // odd n: the shifts are the ramps
    MixedArgs a = p->mx;
    a.in = src;
    a.out = dst;
    a.flip = 0;
    a.pre = p->shift == 1 ? p->mx_shift : p->shift == 2 ? p->mx_ishift : nullptr;
    const RaderArgs rd{p->rd_conv, reinterpret_cast<const int2*>(p->rd_perm), (int)p->n};
    e = launch_rader(a, rd, stream);
  } else if (p->bmixed) {
    MixedArgs a = p->mx;
    a.in = src;
    a.out = dst;
    a.flip = 0;
    a.pre = p->shift == 1 ? p->chirp_shift : p->shift == 2 ? p->chirp_ishift : p->chirp;
    const ChirpMixedArgs c{p->bhat, p->chirp, (int)p->n};
    e = launch_bluestein_mixed(a, c, stream);
  } else if (p->bluestein && p->fourstep) {
    const float2* pre = p->shift == 1 ? p->chirp_shift : p->shift == 2 ? p->chirp_ishift : p->chirp;
    const int64_t m = p->bm;
    float2* s1 = sc;
    float2* s2 = sc + m * p->batch;
    // pass 1: the chirped row (zero beyond n), forward n2-point column
    // transforms with the four-step factor, into s1
    FourStepArgs f1{src, s1, p->tw_b, p->thi, p->tlo, p->batch, p->n1, p->n2, p->bits, 0,
                    pre, nullptr, p->n, 0, (int)p->n, 0};
    e = launch_fourstep_cols(p->n2, -1, f1, stream, true);
    // pass 2: rows through the forward n1-point transform, times bhat, the
    // inverse n1-point transform and its factor, into s2
    if (e == hipSuccess) {
      FourStepArgs f2{s1, s2, p->tw_a, p->thi, p->tlo, p->batch, p->n1, p->n2, p->bits, 0, p->bhat_t};
      e = launch_chirp_mid(p->n1, f2, stream);
    }
    // pass 3: inverse n2-point column transforms, the first n outputs times c_k, into out
    if (e == hipSuccess) {
      FourStepArgs f3{s2, dst, p->tw_b, p->thi, p->tlo, p->batch, p->n1, p->n2, p->bits, 0,
                      nullptr, p->chirp, 0, p->n, 0, (int)p->n, s1};  // s1 is free after pass 2
      e = launch_chirp_out(p->n2, f3, stream);
    }
  } else if (p->bluestein) {
    const float2* pre = p->shift == 1 ? p->chirp_shift : p->shift == 2 ? p->chirp_ishift : p->chirp;
    BluesteinArgs a{src, dst, p->tw_a, pre, p->chirp, p->bhat, p->batch, (int)p->n};
    e = launch_bluestein(p->bm, a, stream);
  } else if (p->kind == FFT_C2C && p->dims == 1 && !p->fourstep) {
    RowsArgs a{src, dst, p->tw_a, p->batch, p->shift ? 1 : 0, 1, 1};
    e = launch_c2c_rows((int)p->n, p->sign, a, stream);
  } else if (p->kind == FFT_C2C && p->dims == 1) {
    FourStepArgs a{src, sc, p->tw_b, p->thi, p->tlo, p->batch, p->n1, p->n2, p->bits, p->shift};
    e = launch_fourstep_cols(p->n2, p->sign, a, stream);
    if (e == hipSuccess) {
      FourStepArgs b{sc, dst, p->tw_a, p->thi, p->tlo, p->batch, p->n1, p->n2, p->bits, 0};
      e = launch_fourstep_rows(p->n1, p->sign, b, stream);
    }
  } else if (p->kind == FFT_C2C && !p->tall) {
    RowsArgs a{src, dst, p->tw_a, p->batch * p->ny, p->shift ? 2 : 0, p->ny, 0};
    e = launch_c2c_rows((int)p->nx, p->sign, a, stream);
    if (e == hipSuccess) {
      ColsArgs c{dst, dst, p->tw_b, p->ny, p->nx, p->batch};
      e = launch_c2c_cols((int)p->ny, p->sign, c, stream);
    }
  } else if (p->kind == FFT_C2C && p->fold) {
    // rows and the first column factor: in -> scratch; columns: scratch -> out
    FoldArgs a{src, dst, sc, p->tw_ca, p->tw_cb, p->wt, p->batch, p->ny, p->nx, p->shift ? 1 : 0};
    e = launch_fold_2d(p->sign, a, stream);
  } else if (p->kind == FFT_C2C) {
    // rows: in -> scratch; column step A in place on scratch; step B scratch -> out
    const uint32_t nx = (uint32_t)p->nx, na = kTallSplit, nb = (uint32_t)(p->ny / kTallSplit);
    RowsArgs a{src, sc, p->tw_a, p->batch * p->ny, p->shift ? 2 : 0, p->ny, 0};
    e = launch_c2c_rows((int)p->nx, p->sign, a, stream);
    if (e == hipSuccess) {
      ColStageArgs ca{sc, sc, p->tw_ca, p->wt, (int64_t)na * nx, p->ny * p->nx, (int)p->batch,
                      nx, (uint32_t)ilog2c(nx), nx, na * nx, nx, na * nx};
      e = launch_col_stage((int)nb, p->sign, true, ca, stream);
    }
    if (e == hipSuccess) {
      ColStageArgs cb{sc, dst, p->tw_cb, p->wt, (int64_t)nb * nx, p->ny * p->nx, (int)p->batch,
                      nx, (uint32_t)ilog2c(nx), na * nx, nx, nx, nb * nx};
      e = launch_col_stage((int)na, p->sign, false, cb, stream);
    }
  } else if (is_direct(p->kind)) {
    DirectArgs a{in, out, p->trig, p->batch, (int)p->n, (int)p->mmax, p->spec_layout};
    e = launch_direct(p->kind == FFT_C2R_DIRECT, a, stream);
  } else {
    if (p->real_pairs) {
      RealArgs a{in, out, p->tw_full, p->rt, p->batch, (int)p->mmax, p->spec_layout};
      e = p->kind == FFT_R2C ? launch_r2c_pairs((int)p->n, a, stream) : launch_c2r_pairs((int)p->n, a, stream);
    } else {
      RealArgs a{in, out, p->tw_a, p->rt, p->batch, (int)p->mmax, p->spec_layout};
      e = p->kind == FFT_R2C ? launch_r2c((int)(p->n / 2), a, stream) : launch_c2r((int)(p->n / 2), a, stream);
    }
  }
  if (e != hipSuccess) return hip_err(e, "kernel launch");
  return FFT_OK;
}

// fft_exec and fft_exec_noalloc after their argument checks: the plan's
// device made current, ordering against the plan's previous exec, the
// launches, and the completion event.  Outside graph capture every kernel of
// the exec binds the plan's event to its own completion (exec_done_event,
// FFTAMD_LAUNCH), so the event ends up standing for the exec's last kernel;
// fft_plan_destroy waits for it, and an exec on another stream than the
// plan's last one first waits for it (both would use the plan's scratch).
// The inner plans of an exec (any-length 2D and real plans) bind the outer
// plan's event.  Inside a capture none of this is done (an event bound
// outside the capture cannot be waited on inside it): the caller orders
// captured work and finishes the graph's launches before destroying the
// plan.
int exec_common(fft_plan* p, const void* in, void* out, fft_stream_t stream_, float2* sc) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_err(e, "hipGetDevice");
  if (cur != p->device) {
    e = hipSetDevice(p->device);
    if (e != hipSuccess) return hip_err(e, "hipSetDevice");
  }
  hipEvent_t& bound = exec_done_event();
  const hipEvent_t outer = bound;  // non-null while an outer plan's exec runs this one
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const bool capturing = hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
  const bool track = !capturing && !outer;
  int rc = FFT_OK;
  if (track && p->recorded && p->last_stream != stream) {
    e = hipStreamWaitEvent(stream, p->done, 0);
    if (e != hipSuccess) rc = hip_err(e, "hipStreamWaitEvent");
  }
  if (rc == FFT_OK) {
    if (track) bound = p->done;
    rc = run_plan(p, in, out, stream_, sc);
    bound = outer;
    if (track) {
      // also after a failed sequence: its first kernels may have been
      // enqueued (an event nothing was bound to completes at once)
      p->recorded = true;
      p->last_stream = stream;
    }
  }
  if (rc == FFT_OK) p->executed = true;  // only once a launch sequence went through
  if (cur != p->device) (void)hipSetDevice(cur);
  return rc == FFT_OK ? ok() : rc;
}

// Scratch the inner plans of p own (an any-length 2D or real plan runs its
// complex transforms through inner plans).
size_t inner_scratch_bytes(const fft_plan* p) {
  size_t b = 0;
  for (const fft_plan* q : {p->inner, p->inner2})
    if (q) b += q->scratch_bytes + inner_scratch_bytes(q);
  return b;
}

// ---------------------------------------------------------------------------
// Static scratch of fft_exec_noalloc: one array per device, part of the
// library's device code (allocated when the code object is loaded on a
// device, held until the process ends).  Host code never uses the array's
// name as an address: the device address comes from hipGetSymbolAddress,
// once per device, with that device current.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = FFT_NOALLOC_MAX_SCRATCH_BYTES;
constexpr int kStaticScratchDevices = 64;

}  // namespace

static __device__ __align__(256) float2 scratch[kStaticScratchBytes / sizeof(float2)];

namespace {

std::mutex g_static_mu;
float2* g_static_ptr[kStaticScratchDevices] = {};

int static_scratch(int dev, float2** out) {
  if (dev < 0 || dev >= kStaticScratchDevices)
    return set_err(FFT_ENOTSUP, "fft_exec_noalloc supports device ordinals below 64");
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_err(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_err(e, "hipSetDevice");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) return hip_err(e, "hipGetSymbolAddress(static scratch)");
    if (!ptr) return set_err(FFT_EHIP, "hipGetSymbolAddress(static scratch) returned NULL");
    g_static_ptr[dev] = static_cast<float2*>(ptr);
  }
  *out = g_static_ptr[dev];
  return FFT_OK;
}

}  // namespace

extern "C" {

int fft_exec(fft_plan* p, const void* in, void* out, fft_stream_t stream) {
  if (check_exec_args(p, in, out) != FFT_OK) return g_err.code;
  return exec_common(p, in, out, stream, p->scratch);
}

int fft_exec_noalloc(fft_plan* p, const void* in, void* out, fft_stream_t stream) {
  if (check_exec_args(p, in, out) != FFT_OK) return g_err.code;
  if (inner_scratch_bytes(p))
    return set_err(FFT_ENOTSUP, "fft_exec_noalloc: the plan's inner transforms own scratch of their own");
  if (p->scratch_bytes > kStaticScratchBytes)
    return set_err(FFT_ENOTSUP, "fft_exec_noalloc: the plan needs " + std::to_string(p->scratch_bytes) +
                                    " bytes of scratch, the static buffer holds " +
                                    std::to_string(kStaticScratchBytes));
  float2* sc = nullptr;
  if (p->scratch_bytes && static_scratch(p->device, &sc) != FFT_OK) return g_err.code;
  return exec_common(p, in, out, stream, sc);
}

void fft_plan_destroy(fft_plan* p) {
  if (!p) {
    ok();
    return;
  }
  // work enqueued with this plan may still read its tables and scratch: wait
  // for its last recorded exec (not for the rest of the device), then free
  // on the plan's device (restoring the caller's)
  wait_plan(p);
  int cur = -1;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  const bool other = have_cur && cur != p->device;
  if (other) (void)hipSetDevice(p->device);
  free_plan(p);
  if (other) (void)hipSetDevice(cur);
  ok();
}

int fft_last_error(const char** msg) {
  if (msg) *msg = g_err.msg.c_str();
  return g_err.code;
}

int64_t fft_max_single_pass_length(void) { return kMaxSinglePass; }

}  // extern "C"
