// launch.hpp -- host-side launchers of the transform kernels (internal API of
// libfft_amd.so; the public C ABI is include/fft.h).
//
// Every launcher picks the kernel instantiated for the given length and sign,
// checks that the length is one it was built for, launches it on `stream`
// and returns the launch status.  Pointers are device pointers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fftamd {

// Completion event of the plan whose kernels are being enqueued: set by
// fft_exec around a plan's launch sequence (outside graph capture), null
// otherwise (thread-local).  Every launch binds it to the completion of its
// own dispatch (the stop event of hipExtLaunchKernel), so after an exec it
// stands for the end of the exec's last kernel without a separate marker
// command in the stream (a marker per exec measured 1-2 us of idle GPU time
// between launches).
hipEvent_t& exec_done_event();
#define FFTAMD_LAUNCH(KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                   \
  hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, nullptr, ::fftamd::exec_done_event(), 0, \
                        __VA_ARGS__)

// Whole rows of length n (contiguous), one transform per row.
// shift_mode: 0 none; 1 multiply element j by (-1)^j; 2 multiply element j of
// row r by (-1)^(r mod rows_per_image + j) (2D chessboard).
struct RowsArgs {
  const float2* in;
  float2* out;
  const float2* tw;  // single-pass stage table for n
  int64_t rows;
  int shift_mode;
  int64_t rows_per_image;
  int stream_store;  // 1: non-temporal stores (output not re-read soon)
};
hipError_t launch_c2c_rows(int n, int sign, const RowsArgs& a, hipStream_t stream);

// Columns of [images][ny][nx]: transform of length ny over every column, with
// element stride nx.  In place is allowed (in == out).
struct ColsArgs {
  const float2* in;
  float2* out;
  const float2* tw;  // single-pass stage table for ny
  int64_t ny, nx, images;
  int shift;  // 1: multiply row i by (-1)^i on load (the shift along y; ny even)
};
hipError_t launch_c2c_cols(int ny, int sign, const ColsArgs& a, hipStream_t stream);

// Real transforms of length n = 2h through one complex transform of length h.
// R2C: in float [rows][2h] -> out complex, bins 0..mmax.
// C2R: in complex bins 0..mmax -> out float [rows][2h].
// Spectrum layout: mmajor = 0 -> [rows][mmax+1]; 1 -> [mmax+1][rows].
struct RealArgs {
  const void* in;
  void* out;
  const float2* tw;  // single-pass stage table for h
  const float2* rt;  // e^{-2 pi i k/n}, k = 0..h
  int64_t rows;
  int mmax;
  int mmajor;
};
hipError_t launch_r2c(int h, const RealArgs& a, hipStream_t stream);
hipError_t launch_c2r(int h, const RealArgs& a, hipStream_t stream);
// Two real rows per complex transform of the full length n (rows even;
// tw: the stage table for n; rt unused).
hipError_t launch_r2c_pairs(int n, const RealArgs& a, hipStream_t stream);
hipError_t launch_c2r_pairs(int n, const RealArgs& a, hipStream_t stream);

// Four-step transform of length n = n1*n2 (element n1 + N1*n2 -> bin
// k2 + N2*k1).  Pass 1 (columns): in -> scratch, length-n2 transforms over
// stride n1, each output multiplied by W_n^{n1*k2}.  Pass 2 (rows): scratch ->
// out, length-n1 transforms over the rows k2, stored transposed.  The scratch
// holds the values in blocks sized to both passes' workgroups (kernels.hpp,
// fs_block_index); n1 must be n2 or n2/2.
// W_n^e = thi[e >> bits] * tlo[e & (2^bits - 1)].
struct FourStepArgs {
  const float2* in;
  float2* out;
  const float2* tw;   // stage table (n2 for pass 1, n1 for pass 2)
  const float2* thi;
  const float2* tlo;
  int64_t batch;
  int n1, n2, bits;
  int shift;  // pass 1 only: multiply element j by (-1)^j (1D chessboard)
  // The hooked pass 1 (hook = true in launch_fourstep_cols), for the chirp
  // transform: it reads rows of in_len values in_stride apart (zero beyond
  // in_len) and multiplies element j by pre[j] (if set).  The chirp passes
  // after it (launch_chirp_mid/out) use pre, post, out_stride, out_len and
  // sink as described there.  Other passes ignore these fields.
  const float2* pre;
  const float2* post;
  int64_t in_stride, out_stride;
  int in_len, out_len;
  float2* sink;  // launch_chirp_out: >= 1024 elements nothing else reads (dropped outputs land there)
  int64_t stagger;  // set by the launcher: wall-clock ticks by which half of the workgroups start late
};
hipError_t launch_fourstep_cols(int n2, int sign, const FourStepArgs& a, hipStream_t stream, bool hook = false);
hipError_t launch_fourstep_rows(int n1, int sign, const FourStepArgs& a, hipStream_t stream);
// The chirp transform above m = 16384 after its first four-step pass
// (k_chirp.hip), on FourStepArgs of the length m = n1*n2:
// launch_chirp_mid: rows k2 of pass 1's block layout (in) through the
//   forward n1-point transform, times pre[k2*n1 + k1] (the chirp's transform
//   at bin k2 + n2*k1), the inverse n1-point transform and W_m^{-j1*k2};
//   rows stored contiguously to out as [batch][n2][n1].  tw: stage table of
//   n1 (tposed_values); thi/tlo/bits: the two-level table of m.
// launch_chirp_out: columns j1 of in ([batch][n2][n1]) through the inverse
//   n2-point transform over k2; output j = j1 + n1*j2 kept for j < out_len,
//   times post[j], written to row b of out (out_stride apart); outputs past
//   out_len are written to sink instead.  tw: stage table of n2 (cols_values).
hipError_t launch_chirp_mid(int n1, const FourStepArgs& a, hipStream_t stream);
hipError_t launch_chirp_out(int n2, const FourStepArgs& a, hipStream_t stream);

// One step of a column transform split in two (2D column pass of tall images,
// ny = na * nb; column row index i = ia + na*ib, output k = kb + nb*ka).
// Lines c = 0 .. nlines-1 of each image; with q = c / nx and r = c % nx the
// line's elements sit at q*a_in + r + t*s_in (t < L) and its results go to
// q*a_out + r + k*s_out.  Step A (L = nb): q = ia, elements ia + na*ib, each
// output multiplied by W_ny^{ia*kb} (wt[e] = e^{-2 pi i e/ny}), stored in
// place.  Step B (L = na): q = kb, elements na*kb + ia, stored at row kb + nb*ka.
struct ColStageArgs {
  const float2* in;
  float2* out;
  const float2* tw;   // stage table for L
  const float2* wt;   // W_ny table (step A only)
  int64_t nlines;     // lines per image
  int64_t image_stride;
  int images;
  uint32_t nx, log2nx;
  uint32_t a_in, s_in, a_out, s_out;
};
hipError_t launch_col_stage(int len, int sign, bool twiddle, const ColStageArgs& a, hipStream_t stream);

// Tall 2D images [images][ny][nx] in two passes (k_fold.hip), for the shapes
// fold_supported() accepts; na = fold_na(ny, nx), nb = ny / na.  Pass 1: rows
// yb + nb*ya (ya < na) transformed along x, the na-point DFT across them,
// output ka times W_ny^{yb*ka}, stored as row ka of group yb of scratch
// (groups of na adjacent rows, fold_group_pitch(nx, na) elements apart).
// Pass 2: nb-point transforms over row ka of every group, stored to rows
// ka + na*j of out (natural order).  in may equal out; scratch must not
// overlap either.
struct FoldArgs {
  const float2* in;
  float2* out;
  float2* scratch;    // fold_scratch_elems(ny, nx, images) elements
  const float2* tw;   // stage table of nx, fold_row_values(nx, na) values per thread
  const float2* tw2;  // stage table of nb, fold_col_values(nb, fold_c(nb)) values per thread
  const float2* wy;   // e^{-2 pi i e/ny}, e < ny
  int64_t images;
  int64_t ny, nx;
  int shift;          // 1: (-1)^(y + x) on the load (fftshift of both axes)
  int64_t stagger;    // set by the launcher: wall-clock ticks by which half of the workgroups start late
};
bool fold_supported(int64_t ny, int64_t nx);
hipError_t launch_fold_2d(int sign, const FoldArgs& a, hipStream_t stream);

// C2C rows whose length n <= kMaxMixedLength has no prime factor above 13:
// mixed-radix Stockham stages of radix 2, 3, 4, 5, 7 or 8 (schedule chosen at
// plan time), the line resident in LDS between stages.  Stage s has radix
// radix[s], ns[s] = product of the radices before it, m[s] = n / radix[s]
// butterflies, and its twiddles W_{ns*radix}^{r*j} at tw[twoff[s] + (r-1)*ns + j].
// ns_magic[s] = ceil(2^32 / ns[s]), so that b / ns = umulhi(b, ns_magic) for
// b < 2^16.  pre: n factors applied on load (the shift ramps), or null.
// Threads: tpl per line, lines per workgroup; each thread takes butterflies
// t, t + tpl, ..., at most kb per stage (kb = 2, kMixedButterflies, with
// radices up to 8 for n <= 8192 and up to 16 above; kb = 1 with radices up
// to 16: 2..8, 10..16), so tpl * kb >= m[s] and every stage needs
// m[s] <= 1024 * kb.  One line of n <= 16384 complex values fits the LDS.
constexpr int kMaxMixedLength = 16384;
constexpr int kMixedMaxStages = 16;
constexpr int kMixedButterflies = 2;
struct MixedArgs {
  const float2* in;
  float2* out;
  const float2* tw;
  const float2* pre;
  int64_t rows;
  int n, nstages, tpl, lines, kb;
  int flip;  // 1: negate the elements of odd index on load (exact sign flip; the shift of even n)
  int pad;  // LDS line: 1 = one pad element after every 32 elements, 0 = none
  int radix[kMixedMaxStages];
  int ns[kMixedMaxStages];
  int m[kMixedMaxStages];
  int twoff[kMixedMaxStages];
  uint32_t ns_magic[kMixedMaxStages];
};
hipError_t launch_mixed(int sign, const MixedArgs& a, hipStream_t stream);

// Column transforms of a mixed-radix length n = a.n over [images][n][nx]
// (the column pass of 2D plans whose ny has a mixed-radix schedule):
// a.in / a.out hold the images (in place allowed: a workgroup reads its whole
// tile before writing it), a.pre / a.flip the shift along y on load; the
// schedule, tables and threads per line of `a` as for launch_mixed (a.rows
// unused; a.lines is set by the launcher to the columns per workgroup).
// n * nx must stay below 2^29 (32-bit element offsets within an image).  mixed_cols_tile(a) adjacent columns per workgroup
// are staged in LDS (rows of the tile are runs of 8 * columns bytes), the
// stages run on the lines in LDS a group of lines at a time, and the columns
// are stored back.
struct MixedColsArgs {
  int64_t nx, images;
  // optional (thi non-null): the stored value of row k of column x is
  // multiplied by W^{x k} = thi[e >> bits] * tlo[e & (2^bits - 1)], e = x k
  // (x k < 2^32; the four-step of lengths with no prime factor above 13)
  const float2* thi;
  const float2* tlo;
  int bits;
  // launch_mixed_rows_t only: the rotation of the transposed store
  int64_t rot;
};
// columns per workgroup (16 while they take at most 80 KiB of LDS and 16
// lines at most 384 threads, else 8), or 0 when not even 8 fit (the caller
// then transposes instead)
int mixed_cols_tile(const MixedArgs& a);
hipError_t launch_mixed_cols(int sign, const MixedArgs& a, const MixedColsArgs& c, hipStream_t stream);
// The same tiles over rows: a.in holds c.images * c.nx contiguous rows of
// n = a.n values; each image of c.nx rows [c.nx][n] is transformed along
// its rows and stored transposed, [n][c.nx], rotated by c.rot (0 <= rot <
// n * nx: element e of an output image goes to (e + rot) mod (n * nx)).
// The second pass of the four-step of smooth lengths (rows of n1, the
// output index k1 * n2 + k2).  a.out must not overlap a.in.
hipError_t launch_mixed_rows_t(int sign, const MixedArgs& a, const MixedColsArgs& c, hipStream_t stream);

// C2C rows of a prime length p by Rader's algorithm ("High Performance
// Fourier Transforms on GPUs with GLSL", section 2.3, names it beside
// Bluestein's for prime lengths; the steps below are the textbook form):
// with g a generator of the nonzero residues mod p and N = p - 1,
//   X_(g^q) = x_0 + sum_r x_(g^-r) w^(g^(q - r)),  X_0 = x_0 + sum_(j>0) x_j,
// a cyclic convolution of length N done with the mixed-radix stages of `a`
// (a schedule of N, kb = 1; a.in / a.out hold rows of p values).
//   conv: the forward N-point transform of b_m = w^(g^m) divided by N (w =
//         e^{sign 2 pi i/p}; the sign of the transform lives here);
//   perm: for j = 1 .. p-1, .x = position of x_j in the convolution input
//         ((N - ind j) mod N), .y = index of the convolution output that
//         X_j takes (ind j), with g^(ind j) = j.
// a.pre (the shift of odd lengths) multiplies the input on load.
struct RaderArgs {
  const float2* conv;
  const int2* perm;
  int p;
};
hipError_t launch_rader(const MixedArgs& a, const RaderArgs& rd, hipStream_t stream);

// Bluestein's chirp transform (below) with a convolution length m that is
// not a power of two: the mixed-radix stages of `a` (a schedule of m, kb = 1;
// a.in / a.out hold rows of n values, a.pre the n chirp factors applied on
// load) run on a line of m values in LDS; bhat: the m factors between the
// two transforms; post: the n factors applied on store.
struct ChirpMixedArgs {
  const float2* bhat;
  const float2* post;
  int n;
};
hipError_t launch_bluestein_mixed(const MixedArgs& a, const ChirpMixedArgs& c, hipStream_t stream);

// C2C rows of any length n (2 <= n <= kMaxBluesteinLength) by Bluestein's
// chirp: with c_j = e^{sign pi i j^2/n}, y_k = c_k * (a conv b)_k, where
// a_j = x_j pre_j (pre_j = c_j, times the shift ramp when requested) padded
// with zeros to m >= 2n - 1 and b = conj(c) wrapped around; the convolution
// is inverse_FFT_m(forward_FFT_m(a) * bhat) with bhat = forward_FFT_m(b)/m.
// Rows of n complex64 values, contiguous; in place allowed.
constexpr int kMaxBluesteinLength = 16384;  // m <= 32768: one workgroup per row
// longer lengths run the same computation in three passes (the hooked
// launch_fourstep_cols, launch_chirp_mid, launch_chirp_out), up to this length
constexpr int64_t kMaxBluesteinLengthLarge = int64_t(1) << 22;
struct BluesteinArgs {
  const float2* in;
  float2* out;
  const float2* tw;    // stage table for m (forward)
  const float2* pre;   // n factors applied on load
  const float2* post;  // n factors applied on store (c_k)
  const float2* bhat;  // m factors between the two transforms
  int64_t rows;
  int n;
};
hipError_t launch_bluestein(int m, const BluesteinArgs& a, hipStream_t stream);

// Real transforms of lengths that are not powers of two: the complex
// transform runs on an any-length C2C plan (mixed radix or chirp); these
// element-wise kernels do the packing around it ("fourier.ts" header and
// fftAnalysRealWGSL / fftSynthRealWGSL for even n = 2h; the definition of the
// real transform for odd n).  Spectrum: bins 0..mmax, [rows][mmax+1] or
// [mmax+1][rows] when mmajor.  rt: e^{-2 pi i k/n}, k = 0..n/2.
struct RealAnyArgs {
  const void* in;
  void* out;
  const float2* rt;
  int64_t rows;
  int n, len, mmax, mmajor;  // len: complex row length of the scratch (n/2 or n)
};
// even n: Z = FFT_h(x viewed as h complex) -> bins (Xe + W^k Xo)
hipError_t launch_real_unpack(const RealAnyArgs& a, hipStream_t stream);
// even n: bins -> Z (Hermitian assembly), then inverse FFT_h gives x as h complex
hipError_t launch_real_pack(const RealAnyArgs& a, hipStream_t stream);
// odd n: x -> (x, 0); FFT_n -> bins 0..mmax; bins -> full Hermitian row; Re of a row
hipError_t launch_real_complexify(const RealAnyArgs& a, hipStream_t stream);
hipError_t launch_real_extract(const RealAnyArgs& a, hipStream_t stream);
hipError_t launch_real_hermitian(const RealAnyArgs& a, hipStream_t stream);
hipError_t launch_real_part(const RealAnyArgs& a, hipStream_t stream);

// Transpose of `images` complex64 matrices [rows][cols] -> [cols][rows]
// (out must not overlap in), through 32 x 32 LDS tiles so both sides are
// coalesced.  Used by 2D plans with an axis that is not a power of two, and
// by the four-step of smooth lengths, whose fftshift is the rotation rot
// (0 <= rot < rows * cols): element e of an output image goes to
// (e + rot) mod (rows * cols).
hipError_t launch_transpose(const float2* in, float2* out, int64_t rows, int64_t cols, int64_t images,
                            hipStream_t stream, int64_t rot = 0);

// Band-limited direct transforms (any n, 2 <= n <= kMaxDirectLength):
// analysis reads real rows [rows][n] (float) and writes bins 0..mmax;
// synthesis reads bins 0..mmax and writes real rows.  The spectrum is complex
// [rows][mmax+1], or [mmax+1][rows] when mmajor.  trig holds
// e^{-2 pi i u/n} = (cos, -sin)(2 pi u/n) for u = 0..n/2.  Requires 2 mmax < n.
constexpr int kMaxDirectLength = 16384;
struct DirectArgs {
  const void* in;
  void* out;
  const float2* trig;
  int64_t rows;
  int n, mmax, mmajor;
};
hipError_t launch_direct(bool synthesis, const DirectArgs& a, hipStream_t stream);

}  // namespace fftamd
