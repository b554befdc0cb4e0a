/*
 * oracle.c -- plain, slow, double-precision CPU reference for the FFT hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's cpu_baseline leg load this library.  The GPU product path never
 * calls it, and it shares no source, header, table or helper with the HIP
 * library: it computes its own twiddles, in its own file, built by gcc.
 *
 * Everything works on interleaved complex double arrays (re, im, re, im ...).
 *
 * Definitions followed (pages cited by title and section):
 *  - DFT and its sign / normalisation: "High Performance Fourier Transforms on
 *    GPUs with GLSL" (Mota), section 2.2, Equation 5.  Forward uses
 *    e^{-2 pi i jk/N}; the inverse here is the same sum with e^{+...} and is
 *    NOT divided by N (the WGSL Fourier-stage source, turing-sphere fourier.ts,
 *    stockham(): "Unnormalized").
 *  - Fast algorithm: radix-2 decimation in time, same dissertation, section
 *    2.3.1, Equation 9: X_k = E_k + w^k O_k, X_{k+N/2} = E_k - w^k O_k, with E
 *    and O the half-length transforms of the even- and odd-indexed samples.
 *    Applied recursively; the twiddle w^k = e^{sign 2 pi i k/N} is evaluated
 *    directly with libm cos/sin in f64 for each k (one table per length, no
 *    recurrence between entries).
 *  - 2D transform: same dissertation, section 2.7, Equation 19 (row-column
 *    decomposition): transform every row, then every column.
 *  - Real transforms: turing-sphere fourier.ts header comment and
 *    fftAnalysWGSL / fftSynthWGSL: analysis keeps m = 0..mmax of the forward
 *    transform of the real row; synthesis assembles X_0 = Re F_0,
 *    X_m = F_m, X_{N-m} = conj(F_m) (1 <= m <= mmax), zero elsewhere, runs the
 *    inverse and keeps the real part.
 *  - Band-limited direct sums: fourier.ts dftSynthWGSL / dftAnalysWGSL
 *    (O(nphi * mmax) per row), used as an independent cross-check.
 *  - fftshift: "The 1D fftshift in CUDA by chessboard multiplication": the
 *    zero frequency moves to index M = floor(N/2) (M = N/2 for even N, the
 *    page's (N-1)/2 for odd N), i.e. out[i] = Y[(i - M) mod N]; per axis in
 *    2D (even lengths there).
 *  - Lengths that are not powers of two: the definition itself (oracle_dft),
 *    with the factors e^{sign 2 pi i e/n} tabulated once per length for
 *    e = 0..n-1 and indexed by e = (j*k) mod n.
 *
 * Threads: rows (and, in 2D, columns) are split statically over `threads`
 * POSIX threads; threads <= 0 means every online core.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define TWO_PI 6.283185307179586476925286766559

/* ------------------------------------------------------------------------ */
/* threading helper: run fn(ctx, lo, hi) over [0, count) split in contiguous  */
/* chunks                                                                     */
/* ------------------------------------------------------------------------ */
typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);

typedef struct {
  range_fn fn;
  void* ctx;
  int64_t lo, hi;
} range_job;

static void* range_entry(void* p) {
  range_job* j = (range_job*)p;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

static int resolve_threads(int threads) {
  if (threads > 0) return threads;
  long c = sysconf(_SC_NPROCESSORS_ONLN);
  return c > 0 ? (int)c : 1;
}

static void parallel_for(int threads, int64_t count, range_fn fn, void* ctx) {
  threads = resolve_threads(threads);
  if (threads > count) threads = (int)(count > 0 ? count : 1);
  if (threads <= 1) {
    fn(ctx, 0, count);
    return;
  }
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * threads);
  range_job* jobs = (range_job*)malloc(sizeof(range_job) * threads);
  for (int t = 0; t < threads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].lo = count * t / threads;
    jobs[t].hi = count * (t + 1) / threads;
    pthread_create(&tid[t], NULL, range_entry, &jobs[t]);
  }
  for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
  free(tid);
  free(jobs);
}

/* ------------------------------------------------------------------------ */
/* brute-force DFT: the definition written out, O(N^2)                       */
/* ------------------------------------------------------------------------ */
/* y_k = sum_j x_j e^{sign 2 pi i jk/n}.  The exponent j*k is reduced modulo n
 * in integers first, so the angle is exact up to one rounding. */
void oracle_dft_brute(const double* x, double* y, int64_t n, int sign) {
  for (int64_t k = 0; k < n; ++k) {
    double sr = 0.0, si = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      int64_t e = (j * k) % n;
      double a = TWO_PI * (double)e / (double)n;
      double c = cos(a), s = sign * sin(a);
      double xr = x[2 * j], xi = x[2 * j + 1];
      sr += xr * c - xi * s;
      si += xr * s + xi * c;
    }
    y[2 * k] = sr;
    y[2 * k + 1] = si;
  }
}

/* The same definition for a batch of rows of any length n >= 1, with the
 * factors tabulated once: w[e] = e^{sign 2 pi i e/n}, e = 0..n-1, each from
 * libm cos/sin of an exactly reduced angle, and y_k = sum_j x_j w[(j*k) mod n].
 * O(n^2) per row; rows x bins are split over the threads. */
typedef struct {
  const double* x;
  double* y;
  const double* w;
  int64_t n;
} dft_ctx;

static void dft_body(void* p, int64_t lo, int64_t hi) {
  const dft_ctx* c = (const dft_ctx*)p;
  const int64_t n = c->n;
  for (int64_t t = lo; t < hi; ++t) {
    const int64_t row = t / n, k = t % n;
    const double* x = c->x + 2 * row * n;
    double sr = 0.0, si = 0.0;
    int64_t e = 0; /* (j*k) mod n, advanced by k per term */
    for (int64_t j = 0; j < n; ++j) {
      const double wr = c->w[2 * e], wi = c->w[2 * e + 1];
      const double xr = x[2 * j], xi = x[2 * j + 1];
      sr += xr * wr - xi * wi;
      si += xr * wi + xi * wr;
      e += k;
      if (e >= n) e -= n;
    }
    c->y[2 * (row * n + k)] = sr;
    c->y[2 * (row * n + k) + 1] = si;
  }
}

int oracle_dft(const double* x, double* y, int64_t n, int64_t batch, int sign, int threads) {
  if (n < 1 || batch < 1 || (sign != 1 && sign != -1) || x == y) return -1;
  double* w = (double*)malloc(sizeof(double) * 2 * (size_t)n);
  if (!w) return -2;
  for (int64_t e = 0; e < n; ++e) {
    const double a = TWO_PI * (double)e / (double)n;
    w[2 * e] = cos(a);
    w[2 * e + 1] = sign * sin(a);
  }
  dft_ctx c = {x, y, w, n};
  parallel_for(threads, batch * n, dft_body, &c);
  free(w);
  return 0;
}

/* Selected outputs of the same definition, one sum per requested bin:
 * y[q] = sum_j x_j e^{sign 2 pi i j*bins[q]/n}, O(n) each, for checking
 * transforms too long for a full oracle run.  Rows of `threads` threads split
 * the sum; the partial sums are added in a fixed order. */
typedef struct {
  const double* x;
  int64_t n, k;
  int sign;
  int parts;
  double* acc; /* [parts][2] */
} bin_ctx;

static void bin_body(void* p, int64_t lo, int64_t hi) {
  bin_ctx* c = (bin_ctx*)p;
  for (int64_t part = lo; part < hi; ++part) {
    int64_t j0 = c->n * part / c->parts, j1 = c->n * (part + 1) / c->parts;
    double sr = 0.0, si = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
      /* j*k mod n without overflow: n <= 2^31 keeps the product in int64 */
      int64_t e = (int64_t)(((__int128)j * c->k) % c->n);
      double a = TWO_PI * (double)e / (double)c->n;
      double co = cos(a), sn = c->sign * sin(a);
      double xr = c->x[2 * j], xi = c->x[2 * j + 1];
      sr += xr * co - xi * sn;
      si += xr * sn + xi * co;
    }
    c->acc[2 * part] = sr;
    c->acc[2 * part + 1] = si;
  }
}

int oracle_dft_bins(const double* x, int64_t n, const int64_t* bins, int64_t nbins, double* y,
                    int sign, int threads) {
  if (n < 1 || nbins < 0 || (sign != 1 && sign != -1)) return -1;
  int parts = resolve_threads(threads) * 4;
  double* acc = (double*)malloc(sizeof(double) * 2 * parts);
  for (int64_t q = 0; q < nbins; ++q) {
    if (bins[q] < 0 || bins[q] >= n) {
      free(acc);
      return -1;
    }
    bin_ctx c = {x, n, bins[q], sign, parts, acc};
    parallel_for(threads, parts, bin_body, &c);
    double sr = 0.0, si = 0.0;
    for (int p = 0; p < parts; ++p) {
      sr += acc[2 * p];
      si += acc[2 * p + 1];
    }
    y[2 * q] = sr;
    y[2 * q + 1] = si;
  }
  free(acc);
  return 0;
}

/* Selected outputs of the 2D definition (Mota, section 2.7, Equation 19
 * written as one double sum): y[q] = sum_{i,j} x[i][j] e^{sign 2 pi i (i*k1/ny
 * + j*k2/nx)} for (k1, k2) = (k1s[q], k2s[q]); O(ny*nx) per output. */
typedef struct {
  const double* x;
  int64_t ny, nx, k1, k2;
  int sign;
  double* acc; /* [ny][2] */
} bin2_ctx;

static void bin2_body(void* p, int64_t lo, int64_t hi) {
  bin2_ctx* c = (bin2_ctx*)p;
  for (int64_t i = lo; i < hi; ++i) {
    double sr = 0.0, si = 0.0;
    const double* row = c->x + 2 * i * c->nx;
    for (int64_t j = 0; j < c->nx; ++j) {
      /* exponent (i*k1*nx + j*k2*ny) / (ny*nx), reduced modulo ny*nx */
      int64_t m = c->ny * c->nx;
      int64_t e = (int64_t)((((__int128)i * c->k1 * c->nx) + ((__int128)j * c->k2 * c->ny)) % m);
      double a = TWO_PI * (double)e / (double)m;
      double co = cos(a), sn = c->sign * sin(a);
      sr += row[2 * j] * co - row[2 * j + 1] * sn;
      si += row[2 * j] * sn + row[2 * j + 1] * co;
    }
    c->acc[2 * i] = sr;
    c->acc[2 * i + 1] = si;
  }
}

int oracle_dft2_bins(const double* x, int64_t ny, int64_t nx, const int64_t* k1s,
                     const int64_t* k2s, int64_t nbins, double* y, int sign, int threads) {
  if (ny < 1 || nx < 1 || nbins < 0 || (sign != 1 && sign != -1)) return -1;
  double* acc = (double*)malloc(sizeof(double) * 2 * ny);
  for (int64_t q = 0; q < nbins; ++q) {
    if (k1s[q] < 0 || k1s[q] >= ny || k2s[q] < 0 || k2s[q] >= nx) {
      free(acc);
      return -1;
    }
    bin2_ctx c = {x, ny, nx, k1s[q], k2s[q], sign, acc};
    parallel_for(threads, ny, bin2_body, &c);
    double sr = 0.0, si = 0.0;
    for (int64_t i = 0; i < ny; ++i) {
      sr += acc[2 * i];
      si += acc[2 * i + 1];
    }
    y[2 * q] = sr;
    y[2 * q + 1] = si;
  }
  free(acc);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* recursive radix-2 decimation in time                                       */
/* ------------------------------------------------------------------------ */
/* w holds e^{sign 2 pi i k/ntop} for k < ntop/2, as (cos, sign*sin) pairs.
 * A sub-transform of length n uses w^{k * ntop/n}. */
static void dit(const double* x, int64_t n, int64_t stride, double* y,
                const double* w, int64_t ntop) {
  if (n == 1) {
    y[0] = x[0];
    y[1] = x[1];
    return;
  }
  int64_t h = n / 2;
  dit(x, h, 2 * stride, y, w, ntop);                /* even samples -> y[0..h) */
  dit(x + 2 * stride, h, 2 * stride, y + 2 * h, w, ntop); /* odd -> y[h..n) */
  int64_t step = ntop / n;
  for (int64_t k = 0; k < h; ++k) {
    double wr = w[2 * (k * step)], wi = w[2 * (k * step) + 1];
    double er = y[2 * k], ei = y[2 * k + 1];
    double orr = y[2 * (k + h)], oi = y[2 * (k + h) + 1];
    double tr = wr * orr - wi * oi;
    double ti = wr * oi + wi * orr;
    y[2 * k] = er + tr;
    y[2 * k + 1] = ei + ti;
    y[2 * (k + h)] = er - tr;
    y[2 * (k + h) + 1] = ei - ti;
  }
}

static double* make_twiddles(int64_t n, int sign) {
  int64_t h = n / 2 > 0 ? n / 2 : 1;
  double* w = (double*)malloc(sizeof(double) * 2 * h);
  for (int64_t k = 0; k < h; ++k) {
    double a = TWO_PI * (double)k / (double)n;
    w[2 * k] = cos(a);
    w[2 * k + 1] = sign * sin(a);
  }
  return w;
}

static int is_pow2(int64_t n) { return n >= 1 && (n & (n - 1)) == 0; }

typedef struct {
  const double* x;
  double* y;
  int64_t n;
  const double* w;
} rows_ctx;

static void rows_body(void* p, int64_t lo, int64_t hi) {
  rows_ctx* c = (rows_ctx*)p;
  for (int64_t r = lo; r < hi; ++r)
    dit(c->x + 2 * r * c->n, c->n, 1, c->y + 2 * r * c->n, c->w, c->n);
}

/* batch rows of length n (power of two), out of place (x != y required). */
int oracle_fft(const double* x, double* y, int64_t n, int64_t batch, int sign,
               int threads) {
  if (!is_pow2(n) || batch < 0 || (sign != 1 && sign != -1) || x == y) return -1;
  double* w = make_twiddles(n, sign);
  rows_ctx c = {x, y, n, w};
  parallel_for(threads, batch, rows_body, &c);
  free(w);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* 2D: every row, then every column (Equation 19)                             */
/* ------------------------------------------------------------------------ */
typedef struct {
  double* y;  /* [batch][ny][nx], transformed in place column by column */
  int64_t ny, nx;
  const double* w;
} cols_ctx;

static void cols_body(void* p, int64_t lo, int64_t hi) {
  cols_ctx* c = (cols_ctx*)p;
  double* col = (double*)malloc(sizeof(double) * 2 * c->ny);
  double* res = (double*)malloc(sizeof(double) * 2 * c->ny);
  for (int64_t q = lo; q < hi; ++q) {
    int64_t b = q / c->nx, j = q % c->nx;
    double* base = c->y + 2 * (b * c->ny * c->nx + j);
    for (int64_t i = 0; i < c->ny; ++i) {
      col[2 * i] = base[2 * i * c->nx];
      col[2 * i + 1] = base[2 * i * c->nx + 1];
    }
    dit(col, c->ny, 1, res, c->w, c->ny);
    for (int64_t i = 0; i < c->ny; ++i) {
      base[2 * i * c->nx] = res[2 * i];
      base[2 * i * c->nx + 1] = res[2 * i + 1];
    }
  }
  free(col);
  free(res);
}

/* columns of a length that is not a power of two: the definition, with the
 * factors e^{sign 2 pi i e/ny} tabulated once (w[e], e = 0..ny-1) */
static void cols_dft_body(void* p, int64_t lo, int64_t hi) {
  cols_ctx* c = (cols_ctx*)p;
  const int64_t ny = c->ny;
  double* col = (double*)malloc(sizeof(double) * 2 * ny);
  for (int64_t q = lo; q < hi; ++q) {
    int64_t b = q / c->nx, j = q % c->nx;
    double* base = c->y + 2 * (b * ny * c->nx + j);
    for (int64_t i = 0; i < ny; ++i) {
      col[2 * i] = base[2 * i * c->nx];
      col[2 * i + 1] = base[2 * i * c->nx + 1];
    }
    for (int64_t k = 0; k < ny; ++k) {
      double sr = 0.0, si = 0.0;
      int64_t e = 0;
      for (int64_t i = 0; i < ny; ++i) {
        const double wr = c->w[2 * e], wi = c->w[2 * e + 1];
        sr += col[2 * i] * wr - col[2 * i + 1] * wi;
        si += col[2 * i] * wi + col[2 * i + 1] * wr;
        e += k;
        if (e >= ny) e -= ny;
      }
      base[2 * k * c->nx] = sr;
      base[2 * k * c->nx + 1] = si;
    }
  }
  free(col);
}

int oracle_fft_2d(const double* x, double* y, int64_t ny, int64_t nx,
                  int64_t batch, int sign, int threads) {
  if (ny < 1 || nx < 1 || batch < 0 || (sign != 1 && sign != -1) || x == y) return -1;
  if (batch == 0) return 0;
  /* rows: the radix-2 transform for powers of two, the definition otherwise */
  int rc = is_pow2(nx) ? oracle_fft(x, y, nx, batch * ny, sign, threads)
                       : oracle_dft(x, y, nx, batch * ny, sign, threads);
  if (rc) return rc;
  if (is_pow2(ny)) {
    double* w = make_twiddles(ny, sign);
    cols_ctx c = {y, ny, nx, w};
    parallel_for(threads, batch * nx, cols_body, &c);
    free(w);
  } else {
    double* w = (double*)malloc(sizeof(double) * 2 * (size_t)ny);
    for (int64_t e = 0; e < ny; ++e) {
      const double a = TWO_PI * (double)e / (double)ny;
      w[2 * e] = cos(a);
      w[2 * e + 1] = sign * sin(a);
    }
    cols_ctx c = {y, ny, nx, w};
    parallel_for(threads, batch * nx, cols_dft_body, &c);
    free(w);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* real transforms (page-3 conventions)                                       */
/* ------------------------------------------------------------------------ */
/* analysis: F[b][m] = (forward FFT of x[b] + 0i)_m for m = 0..mmax.
 * x is [batch][n] real, F is [batch][mmax+1] complex (row-major). */
int oracle_r2c(const double* x, double* F, int64_t n, int64_t batch,
               int64_t mmax, int threads) {
  if (n < 1 || mmax < 0 || mmax > n / 2 || batch < 0) return -1;
  double* xc = (double*)calloc((size_t)(2 * n * batch), sizeof(double));
  double* Y = (double*)malloc(sizeof(double) * 2 * n * batch);
  for (int64_t i = 0; i < n * batch; ++i) xc[2 * i] = x[i];
  /* the radix-2 transform for powers of two, the definition otherwise */
  int rc = batch == 0 ? 0
                      : (is_pow2(n) ? oracle_fft(xc, Y, n, batch, -1, threads)
                                    : oracle_dft(xc, Y, n, batch, -1, threads));
  if (rc == 0)
    for (int64_t b = 0; b < batch; ++b)
      memcpy(F + 2 * b * (mmax + 1), Y + 2 * b * n,
             sizeof(double) * 2 * (mmax + 1));
  free(xc);
  free(Y);
  return rc;
}

/* synthesis: X_0 = Re F_0; X_m = F_m and X_{n-m} = conj F_m for
 * 1 <= m <= mmax; every other bin is zero.  When mmax = n/2 the bin n/2 is
 * its own mirror and takes Re F_{n/2}.  x = Re(inverse FFT(X)), unnormalised.
 * F is [batch][mmax+1] complex (row-major), x is [batch][n] real. */
int oracle_c2r(const double* F, double* x, int64_t n, int64_t batch,
               int64_t mmax, int threads) {
  if (n < 2 || mmax < 0 || mmax > n / 2 || batch < 0) return -1;
  double* X = (double*)calloc((size_t)(2 * n * batch), sizeof(double));
  double* y = (double*)malloc(sizeof(double) * 2 * n * batch);
  for (int64_t b = 0; b < batch; ++b) {
    const double* f = F + 2 * b * (mmax + 1);
    double* row = X + 2 * b * n;
    row[0] = f[0];
    row[1] = 0.0;
    for (int64_t m = 1; m <= mmax; ++m) {
      if (2 * m == n) {
        row[2 * m] = f[2 * m];
        row[2 * m + 1] = 0.0;
        continue;
      }
      row[2 * m] = f[2 * m];
      row[2 * m + 1] = f[2 * m + 1];
      row[2 * (n - m)] = f[2 * m];
      row[2 * (n - m) + 1] = -f[2 * m + 1];
    }
  }
  int rc = batch == 0 ? 0
                      : (is_pow2(n) ? oracle_fft(X, y, n, batch, +1, threads)
                                    : oracle_dft(X, y, n, batch, +1, threads));
  if (rc == 0)
    for (int64_t i = 0; i < n * batch; ++i) x[i] = y[2 * i];
  free(X);
  free(y);
  return rc;
}

/* band-limited direct synthesis (fourier.ts dftSynthWGSL), f64:
 * x[iphi] = Re F_0 + 2 sum_{m=1}^{mmax} Re(F_m e^{+i m phi}), phi = 2 pi iphi/n.
 * Any n >= 1; F is [batch][mmax+1]. */
void oracle_dft_synth_direct(const double* F, double* x, int64_t n,
                             int64_t batch, int64_t mmax) {
  for (int64_t b = 0; b < batch; ++b) {
    const double* f = F + 2 * b * (mmax + 1);
    for (int64_t j = 0; j < n; ++j) {
      double v = f[0];
      for (int64_t m = 1; m <= mmax; ++m) {
        double a = TWO_PI * (double)((m * j) % n) / (double)n;
        v += 2.0 * (f[2 * m] * cos(a) - f[2 * m + 1] * sin(a));
      }
      x[b * n + j] = v;
    }
  }
}

/* band-limited direct analysis (fourier.ts dftAnalysWGSL), f64:
 * F_m = sum_j x_j e^{-i m phi_j} for m = 0..mmax. */
void oracle_dft_analys_direct(const double* x, double* F, int64_t n,
                              int64_t batch, int64_t mmax) {
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t m = 0; m <= mmax; ++m) {
      double sr = 0.0, si = 0.0;
      for (int64_t j = 0; j < n; ++j) {
        double a = TWO_PI * (double)((m * j) % n) / (double)n;
        sr += x[b * n + j] * cos(a);
        si -= x[b * n + j] * sin(a);
      }
      F[2 * (b * (mmax + 1) + m)] = sr;
      F[2 * (b * (mmax + 1) + m) + 1] = si;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* fftshift as an index rotation                                              */
/* ------------------------------------------------------------------------ */
/* idx[i] = (i - M) mod n with M = floor(n/2): out[i] = Y[idx[i]] moves bin 0
 * to index M (n/2 for even n, (n-1)/2 for odd n). */
int oracle_fftshift_index(int64_t n, int64_t* idx) {
  if (n < 1) return -1;
  const int64_t m = n / 2;
  for (int64_t i = 0; i < n; ++i) idx[i] = ((i - m) % n + n) % n;
  return 0;
}

/* The inverse rotation (numpy's ifftshift): idx[i] = (i + M) mod n, M =
 * floor(n/2), which moves index M back to 0.  Equal to the shift above for
 * even n; for odd n the two differ by one place. */
int oracle_ifftshift_index(int64_t n, int64_t* idx) {
  if (n < 1) return -1;
  const int64_t m = n / 2;
  for (int64_t i = 0; i < n; ++i) idx[i] = (i + m) % n;
  return 0;
}

/* out[b][i][j] = y[b][(i - floor(ny/2)) mod ny][(j - floor(nx/2)) mod nx]
 * (complex): the shift of each axis. */
int oracle_fftshift_2d(const double* y, double* out, int64_t ny, int64_t nx,
                       int64_t batch) {
  if (ny < 1 || nx < 1 || y == out) return -1;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t i = 0; i < ny; ++i) {
      int64_t si = ((i - ny / 2) % ny + ny) % ny;
      for (int64_t j = 0; j < nx; ++j) {
        int64_t sj = ((j - nx / 2) % nx + nx) % nx;
        const double* src = y + 2 * ((b * ny + si) * nx + sj);
        double* dst = out + 2 * ((b * ny + i) * nx + j);
        dst[0] = src[0];
        dst[1] = src[1];
      }
    }
  return 0;
}

int oracle_threads(int threads) { return resolve_threads(threads); }
