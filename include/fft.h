/*
 * fft.h -- C ABI of libfft_amd.so: batched fp32 FFTs for AMD Instinct MI355X
 * (gfx950), natural order in and out (Stockham autosort).
 *
 * Conventions
 * -----------
 *  - Transform (DFT definition: "High Performance Fourier Transforms on GPUs
 *    with GLSL", Mota, section 2.2, Equation 5):
 *        y_k = sum_{j=0}^{n-1} x_j * exp(sign * 2*pi*i * j*k / n)
 *    sign = FFT_FORWARD (-1) or FFT_INVERSE (+1).  Neither direction is
 *    normalised (the WGSL Fourier-stage source, turing-sphere fourier.ts,
 *    stockham(), does the same): a forward then an inverse transform returns
 *    n * x.
 *  - Data are fp32.  Complex values are interleaved (re, im) pairs: 8 bytes per
 *    element ("complex64").  Rows are contiguous; batches follow each other.
 *  - C2C lengths: powers of two (single pass up to 16384, four-step up to
 *    2^28), and any other length from 3 to 2^22 (the GLSL dissertation,
 *    section 2.3, names mixed radices and other lengths as the extension of
 *    its radix-2 transforms): lengths up to 16384 with no prime factor above
 *    13 by mixed-radix Stockham stages (radices 2 to 8, 10 to 16) when every
 *    stage has at most 2048 butterflies (one or two per thread); the other
 *    lengths with no prime factor above 13 by a four-step split n = n1 * n2
 *    (n2 <= 1024): n2-point column transforms times the twiddles, n1-point
 *    row transforms, a transpose (three passes through a scratch buffer of
 *    batch * n * 8 bytes); primes p <= 16385 whose p - 1 has a one-kernel
 *    schedule by Rader's algorithm (a cyclic convolution of length p - 1 on
 *    those stages, in one kernel); the others by Bluestein's chirp
 *    transform: two transforms of length m >= 2n - 1 (a power of two, or a
 *    length with a mixed-radix schedule below 1/1.3 of that power of two
 *    when n <= 4096), inside one kernel while m <= 32768 (n <= 16384), else
 *    in three passes (the second holds the inner factors of both transforms)
 *    through a scratch buffer of 2 * batch * m * 8 bytes.
 *  - R2C/C2R lengths: powers of two from 4 to 32768 (one kernel), powers of
 *    two from 65536 to 2^29 and any other length from 3 to 2^22 (fourier.ts
 *    refuses the latter for its FFT; here a complex transform of n/2 values
 *    for even n (the four-step transform for powers of two), with the same
 *    Hermitian pack/unpack as the one-kernel path in separate kernels, or of
 *    n values for odd n, through a plan-owned scratch buffer of
 *    batch * n * 4 bytes (even n) or 2 * batch * n * 8 bytes (odd n)).
 *  - 2D sizes: powers of two from 2 to 16384 (row pass, then column pass),
 *    or any sizes from 2 to 2^22 (at most 65535 images): row transforms,
 *    then the column transforms in place on `out` when ny is a power of two
 *    up to 4096, or has a mixed-radix schedule (see C2C lengths) whose
 *    column tile of 8 or more columns fits the LDS (ny up to about 2560)
 *    and ny * nx <= 2^29; otherwise a tiled transpose, row transforms of the
 *    transposed image and a transpose back, through a plan-owned scratch of
 *    batch * ny * nx * 8 bytes.
 *    The direct kinds below take any length from 2 to 16384.
 *  - Buffers: `in` and `out` are DEVICE pointers owned by the caller, 8-byte
 *    aligned.  The plan owns its twiddle tables and scratch (allocated at
 *    create, freed at destroy).
 *  - Errors: every function records a code and a message, readable with
 *    fft_last_error() from the same host thread.  All argument checks run on
 *    the host before any HIP call.
 *
 * Layouts per kind
 * ----------------
 *  FFT_C2C  in, out: complex64 [batch][n]      (2D: [batch][ny][nx])
 *           in == out (in place) is allowed.
 *  FFT_R2C  in : float32  [batch][n]            (real rows)
 *           out: complex64 [batch][mmax+1]      (row-major, default), or
 *                complex64 [mmax+1][batch]      (m-major, FFT_OPT_SPEC_LAYOUT=1,
 *                the spectrum layout of fourier.ts fftAnalysWGSL)
 *           mmax defaults to n/2 (the full half spectrum, n/2+1 bins).
 *           Only sign = FFT_FORWARD.  in == out is rejected.
 *  FFT_C2R  in : the R2C spectrum layout above (bins 0..mmax)
 *           out: float32 [batch][n]
 *           Bins above mmax are taken as zero; Im of bin 0 (and of bin n/2
 *           when mmax = n/2) is ignored, as fourier.ts fftSynthWGSL does.
 *           Only sign = FFT_INVERSE.  in == out is rejected.
 *           Real transforms follow fourier.ts fftAnalysRealWGSL /
 *           fftSynthRealWGSL: one complex transform of length n/2 plus a
 *           Hermitian pack/unpack (power-of-two n >= 4, and any even n); odd
 *           lengths transform (x, 0) / the full Hermitian row of length n.
 *  FFT_R2C_DIRECT, FFT_C2R_DIRECT
 *           The band-limited direct sums of fourier.ts (dftAnalysWGSL,
 *           dftSynthWGSL), for ANY length 2 <= n <= 16384:
 *             analysis   F_m  = sum_j x_j exp(-2 pi i m j/n),   m = 0..mmax
 *             synthesis  x_j  = Re F_0 + 2 sum_{m=1}^{mmax} Re(F_m exp(+2 pi i m j/n))
 *           Same layouts (and FFT_OPT_SPEC_LAYOUT) as FFT_R2C / FFT_C2R, but
 *           the band limit is strict, 2 mmax < n, as the source requires, and
 *           mmax defaults to floor((n-1)/2).  Im F_0 is ignored.  Cost is
 *           O(n mmax) per row (a real matrix product on the matrix cores);
 *           the cos/sin factors come from a host-f64 table of n entries.
 *           Only FFT_OPT_MMAX and FFT_OPT_SPEC_LAYOUT apply.
 */
#ifndef FFT_AMD_FFT_H
#define FFT_AMD_FFT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fft_plan fft_plan; /* opaque */

/* hipStream_t is `struct ihipStream_t*`; 0 / NULL is the null stream. */
typedef struct ihipStream_t* fft_stream_t;

enum fft_kind { FFT_C2C = 0, FFT_R2C = 1, FFT_C2R = 2, FFT_R2C_DIRECT = 3, FFT_C2R_DIRECT = 4 };
enum fft_sign { FFT_FORWARD = -1, FFT_INVERSE = +1 };

enum fft_status {
  FFT_OK = 0,
  FFT_EINVAL = -1,  /* bad argument: NULL, size < 1, bad kind/sign/option, misaligned */
  FFT_ENOTSUP = -2, /* valid but unsupported: a length this kind does not take, too long */
  FFT_ENOMEM = -3,  /* device allocation failed */
  FFT_EHIP = -4,    /* a HIP runtime call or kernel launch failed (message has details) */
  FFT_ESTATE = -5   /* option set after the first fft_exec */
};

enum fft_option {
  /* 1: multiply the input by (-1)^j in 1D, (-1)^(i+j) in 2D, while loading it,
   * which moves the zero frequency to the middle of the output (the chessboard
   * fftshift: "The 1D fftshift in CUDA by chessboard multiplication").  For
   * power-of-two lengths, and even lengths of the mixed-radix and p * 2^k
   * kernels, the factor is applied by flipping the sign bits of both parts,
   * before any arithmetic, so the result is bitwise the transform of the
   * negated input.  For the other 1D lengths the factor is
   * e^{-sign 2 pi i j floor(n/2)/n}, a table applied on load (folded into the
   * chirp on the chirp-transform path; the page's odd case: a full complex
   * exponential), and bin 0 lands at index floor(n/2) for odd n as well.
   * 2: the inverse rotation (numpy's ifftshift of the output: index floor(n/2)
   * moves to 0), by the factor e^{+sign 2 pi i j floor(n/2)/n}; identical to 1
   * for even lengths (every power-of-two and 2D axis).
   * C2C only; 2D axes are even.  Default 0. */
  FFT_OPT_SHIFT = 1,
  /* R2C: keep bins 0..mmax; C2R: read bins 0..mmax.  0 <= mmax <= n/2
   * (fourier.ts: band limit |m| <= mmax < nphi/2).  Default n/2. */
  FFT_OPT_MMAX = 2,
  /* R2C/C2R (and the direct kinds) spectrum layout: 0 = row-major [batch][mmax+1] (default),
   * 1 = m-major [mmax+1][batch]. */
  FFT_OPT_SPEC_LAYOUT = 3,
  /* R2C/C2R: 1 = transform rows in pairs, rows 2p and 2p+1 as the real and
   * imaginary parts of one complex transform of length n, separated by the
   * even/odd symmetry of the result ("High Performance Fourier Transforms on
   * GPUs with GLSL", section 2.6, Equations 17-18).  0 (default) = each row
   * through a complex transform of length n/2.  Same results up to rounding.
   * Needs an even batch (FFT_EINVAL) and n <= 16384 (FFT_ENOTSUP). */
  FFT_OPT_REAL_PAIRS = 4
};

/*
 * Create a plan for `batch` transforms of length n.
 * n: C2C: a power of two 2 <= n <= 2^28, or any 3 <= n <= 2^22; R2C/C2R: a
 * power of two 4 <= n <= 2^29, or any 3 <= n <= 2^22; the direct kinds: any
 * 2 <= n <= 16384.
 * batch >= 1.
 * kind: enum fft_kind.  sign: FFT_FORWARD or FFT_INVERSE (FFT_FORWARD for the
 * analysis kinds R2C and R2C_DIRECT, FFT_INVERSE for C2R and C2R_DIRECT).
 * Lengths up to 16384 run as one kernel (one workgroup per row, all stages in
 * LDS); longer C2C lengths, up to 2^28, run as two passes (four-step: strided
 * column transforms with the inter-pass twiddle fused into their store, then
 * row transforms with a transposing store) and own a scratch buffer of
 * batch*n*8 bytes.
 * Plans of C2C lengths that are not powers of two own either the mixed-radix
 * stage tables and two shift tables of n entries, or (chirp transform) a
 * stage table of their internal length m (the power of two >= 2n - 1), three
 * chirp tables of n entries and one of m entries, all built in f64 on the
 * host.
 * Direct plans own a table of n/2 + 1 (cos, -sin) pairs.
 * The implementation is chosen here, at plan creation, from the length and
 * the kind, and a length a path cannot take is refused here rather than at
 * execution (the WGSL Fourier-stage source, turing-sphere fourier.ts, header
 * comment: its 'fft' and 'dft' implementations are selected at plan creation,
 * the 'fft' one only for power-of-two lengths whose two workgroup buffers fit
 * the device's workgroup storage; its stockham() throws for other lengths).
 * Here the single-pass limit of 16384 points is what fits the 160 KiB of LDS
 * of one gfx950 workgroup.
 * Uses the current HIP device; the plan stays bound to it.  Returns NULL on
 * error (see fft_last_error).
 */
fft_plan* fft_plan_create(int64_t n, int64_t batch, int kind, int sign);

/*
 * 2D C2C plan over [batch][ny][nx] complex64: every row, then every column
 * (Mota, section 2.7, Equation 19).  ny, nx: powers of two in [2, 16384], or
 * any sizes in [2, 2^22] (then at most 65535 images; the shift options act
 * on each axis).
 * Only kind = FFT_C2C.  For ny in {4096, 8192, 16384} and nx a power of two
 * from 512 with (ny/2048)*nx <= 32768 the transform takes two passes over
 * HBM: na = ny/2048 rows per workgroup transformed along x with the first
 * factor of the column transform fused, then 2048-point column tiles
 * (plan-owned scratch of batch*(ny/na)*(na*nx + 16)*8 bytes).  Other images
 * of 8192 rows and more run the column transform as two steps of
 * 64 x ny/64 points (three passes, scratch of batch*ny*nx*8 bytes); images
 * of 8192 rows and more take at most 65535 images.  The rest transform in
 * place on `out` without scratch.  Returns NULL on error.
 */
fft_plan* fft_plan_create_2d(int64_t ny, int64_t nx, int64_t batch, int kind,
                             int sign);

/* Set an option (enum fft_option).  Only before the first fft_exec of the
 * plan, else FFT_ESTATE.  Returns FFT_OK or an error code. */
int fft_plan_set(fft_plan* plan, int option, int64_t value);

/*
 * Byte sizes the plan reads from `in` and writes to `out` (given its current
 * options).  Either pointer may be NULL.  Returns FFT_OK or FFT_EINVAL.
 */
int fft_plan_get_sizes(const fft_plan* plan, int64_t* in_bytes,
                       int64_t* out_bytes);

/*
 * Enqueue the transform on `stream` and return (asynchronous).  `in` is read,
 * `out` written, both caller-owned device pointers; out-of-place execution
 * never writes `in` (the out-of-place kernel signature (data, out, N) of the
 * "Fast Fourier Transform on CPU and GPU" page, CUDA Kernel: Radix-2 FFT).
 * The direction is the plan's sign, +1 or -1, which flips the exponent of
 * every twiddle factor (the fft_dir uniform of "High Performance Fourier
 * Transforms on GPUs with GLSL", section 3.1, Listing 3.4).
 * The plan's device is made current for the launches and restored after.
 * Outside HIP graph capture, each exec binds a plan-owned event to the
 * completion of its last kernel (no extra command in the stream), and an
 * exec on a different stream than the plan's previous one first makes
 * `stream` wait for that event, so execs of one plan on several streams run
 * one after the other (they share the plan's scratch).  Inside a capture
 * neither is done: the caller orders the captured work and must not replay
 * the graph concurrently with other execs of the plan.
 * Returns FFT_OK, FFT_EINVAL (NULL plan or buffer, misaligned, in == out for
 * R2C/C2R) or FFT_EHIP (launch failure).  The options are locked by the
 * first exec that succeeds; a failed exec leaves them settable.
 */
int fft_exec(fft_plan* plan, const void* in, void* out, fft_stream_t stream);

/* Free the plan.  First waits (hipEventSynchronize) for the event of the
 * plan's last exec outside graph capture, since that work may still read its
 * tables and scratch; work of other plans and streams is not waited for.
 * The plan's device memory comes from the device's stream-ordered pool and
 * goes back to it with hipFreeAsync on the null stream (hipFree would wait
 * for the whole device).
 * A graph that captured an exec of the plan must have finished its launches
 * before the plan is destroyed.  NULL is a no-op. */
void fft_plan_destroy(fft_plan* plan);

/* Code of the last call on this host thread; *msg (if msg is not NULL) points
 * to a thread-local message valid until the next call. */
int fft_last_error(const char** msg);

/* Longest length run as a single kernel (one workgroup per row). */
int64_t fft_max_single_pass_length(void);

/* Size of the static per-device scratch buffer of fft_exec_noalloc, bytes. */
#define FFT_NOALLOC_MAX_SCRATCH_BYTES 268435456

/*
 * fft_exec for callers that cannot allocate device memory at execution time
 * or while capturing a HIP graph, and do not want to keep a scratch buffer
 * per plan: the same kernels and results as fft_exec(plan, in, out, stream),
 * with the plan's intermediate results kept in a buffer of
 * FFT_NOALLOC_MAX_SCRATCH_BYTES (256 MiB) per device that is part of the
 * library's device code (held from the first call on a device until the
 * process ends) instead of the plan's own scratch.  Plans without scratch
 * (single-pass lengths) run as with fft_exec.  It calls no allocating
 * routine: the buffer's device address is looked up once per device, on
 * the first call there.
 * Errors: those of fft_exec, and FFT_ENOTSUP when the plan's scratch
 * (four-step C2C: batch*n*8 bytes; tall 2D and chirp plans: see
 * fft_plan_create and fft_plan_create_2d) exceeds the buffer, or when the
 * plan runs inner plans with scratch of their own (any-length 2D and real
 * plans whose complex transforms need scratch).  Checked before any launch.
 * Every call on one device shares that device's buffer, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that may
 * overlap in time on one device -- on different streams, or on one stream
 * with other work that uses the buffer in between -- race; callers serialise
 * them.
 */
int fft_exec_noalloc(fft_plan* plan, const void* in, void* out, fft_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FFT_AMD_FFT_H */
