// shapes.hpp -- workgroup shapes of the kernels (lines per workgroup, values
// per thread, LDS exchange mode).  Shared by the kernels and by the host code
// that builds each kernel's twiddle table, which depends on the values per
// thread through the radix schedule.
#pragma once

#include "stockham.hpp"

namespace fftamd {

// ---------------------------------------------------------------------------
// workgroup shapes
// ---------------------------------------------------------------------------
constexpr int threads_per_line(int n) { return n / sched_e(n); }
// LDS bytes of c lines of length n (layouts: stockham.hpp RowLds / ColLds)
constexpr int row_lds_bytes(int n, int c, bool split = false, int e = 16, bool xread = false) {
  return row_lds_elems(n, c, split, e, xread) * (split ? 4 : 8);
}
constexpr int col_lds_bytes(int n, int c, bool split = false) {
  return col_lds_elems(n, c, split) * (split ? 4 : 8);
}

// Row lanes: at least 256 threads per workgroup (several short rows share one).
constexpr int rows_per_wg(int n) {
  return threads_per_line(n) >= 256 ? 1 : 256 / threads_per_line(n);
}
// The C2C row kernel: 16 values per thread and a complex LDS exchange, except
// for rows of 4096 and more, which take 32 values per thread and the split
// exchange (half the LDS per line).  For 4096 points that keeps two rows of
// 128 threads per workgroup and eight rows in flight per CU instead of four:
// measured on MI355X (steady state, forward + inverse of 16384 rows) 185.9 -
// 188.0 against 189 - 194 us per launch; 16 values with the split exchange
// (192.9 - 194.5), 32 with the complex one (194.8 - 198.1), 32 with four
// rows per workgroup (255.5) and 64 with one wavefront per row (195.9 -
// 196.3) were slower.  Rows of 8192 and more: one stage fewer, and four
// workgroups fit a CU.
constexpr int kRowsWideMin = 4096;
constexpr int rows_values(int n) { return n >= kRowsWideMin ? 32 : sched_e(n); }
constexpr bool rows_split(int n) { return n >= kRowsWideMin; }
constexpr int rows_threads(int n) { return n / rows_values(n); }
constexpr int rows_lines(int n) { return rows_threads(n) >= 256 ? 1 : 256 / rows_threads(n); }
// Workgroups whose lines are read with a stride (column lanes) or stored
// transposed (row lanes + transposing store) hold up to 16 adjacent lines, so
// every strided access is a run of 16 x 8 B = 128 B.  When 16 values per
// thread with a complex LDS exchange cannot hold enough lines, 64 values per
// thread (<= 512 threads, so up to 256 VGPRs per lane) with the exchange split
// into real and imaginary halves (half the LDS per line) is used instead.
constexpr int kSplitValues = 64;
constexpr bool tile_fits(int n, int e, int c, bool split, bool rowlanes) {
  return e <= n && c * (n / e) <= kMaxThreads &&
         (rowlanes ? row_lds_bytes(n, c, split, e, true) : col_lds_bytes(n, c, split)) <= kLdsBudgetBytes;
}
constexpr int tile_c(int n, int e, bool split, bool rowlanes) {
  int c = 16;
  while (c > 1 && !tile_fits(n, e, c, split, rowlanes)) c /= 2;
  return c;
}
// 1024-point tiles take 32 values per thread and the split exchange (512
// threads, 78 KiB of LDS, two workgroups per CU once the kernels keep to 128
// VGPRs) instead of 16 values and the complex exchange (1024 threads, 130
// KiB, one workgroup per CU).  Per 512 MiB: the four-step of 2^20 488 ->
// 393 us, 2^19 402 -> 366, 2^21 445 -> 415; 2D 1024 x 1024 438 -> 420.
constexpr int kTile1024Values = 32;
constexpr bool tile_split(int n, bool rowlanes) {
  return n == 1024 || (n >= 2 * kSplitValues &&
                       tile_c(n, kSplitValues, true, rowlanes) > tile_c(n, sched_e(n), false, rowlanes));
}
constexpr int tile_e(int n, bool rowlanes) {
  return n == 1024 ? kTile1024Values : tile_split(n, rowlanes) ? kSplitValues : sched_e(n);
}
// waves per SIMD the four-step tile kernels ask the compiler for: 4 (128
// VGPRs, 8-16 B of spills) for the 1024-point tiles, so that two 512-thread
// workgroups share a CU; no bound otherwise
constexpr int fs_waves(int n) { return n == 1024 ? 4 : 1; }
constexpr int tile_lines(int n, bool rowlanes) {
  return tile_c(n, tile_e(n, rowlanes), tile_split(n, rowlanes), rowlanes);
}
// Column-stage kernels (short columns, long runs): about 8192 elements per
// workgroup, up to 64 adjacent lines (512 B runs), 16 values per thread.
constexpr int colstage_lines(int n) {
  int c = 8192 / n;
  if (c > 64) c = 64;
  if (c < 1) c = 1;
  while (c > 1 && (c * threads_per_line(n) > kMaxThreads || col_lds_bytes(n, c) > kLdsBudgetBytes)) c /= 2;
  return c;
}

// values per thread of each kernel family (selects the radix schedule)
constexpr int real_values(int n) { return sched_e(n); }           // k_r2c, k_c2r
constexpr int cols_values(int n) { return tile_e(n, false); }     // k_c2c_cols, k_fs_cols
constexpr int tposed_values(int n) { return tile_e(n, true); }    // k_fs_rows
constexpr int colstage_values(int n) { return sched_e(n); }       // k_col_stage

// Two-pass tall 2D images (k_fold.hip): na rows per pass-1 workgroup (na * nx
// <= 32768 points), column length nb = ny / na = 2048 in pass 2 with 16
// adjacent columns per workgroup (128 B runs), and the values per thread of
// each pass (64 for 32K-point tiles: 512 threads of up to 256 VGPRs).
constexpr int fold_na(int64_t ny, int64_t nx) { return (void)nx, (int)(ny / 2048); }
// The two-pass form: ny in {4096, 8192, 16384} and nx a power of two from
// 512 with a pass-1 tile (fold_na rows of nx) of at most 32768 points
constexpr bool fold_fits(int64_t ny, int64_t nx) {
  return (ny == 4096 || ny == 8192 || ny == 16384) && nx >= 512 && (nx & (nx - 1)) == 0 &&
         fold_na(ny, nx) * nx <= 32768;
}
constexpr int fold_c(int nb) { return (void)nb, 16; }
constexpr int fold_row_values(int nx, int na) { return nx * na >= 32768 ? 64 : 32; }
constexpr int fold_col_values(int nb, int c) { return (void)nb, (void)c, 64; }
// Scratch of the two-pass form: per image nb groups of na adjacent rows, each
// group followed by kFoldPad unused elements, so pass 2's column reads step
// by na*nx + kFoldPad elements instead of a power of two (a power-of-two
// stride keeps each tile's runs on few HBM channels: measured 302 against
// 211 us for the same tile copy).
constexpr int kFoldPad = 16;
constexpr int64_t fold_group_pitch(int64_t nx, int na) { return na * nx + kFoldPad; }
constexpr int64_t fold_scratch_elems(int64_t ny, int64_t nx, int64_t images) {
  return images * (ny / fold_na(ny, nx)) * fold_group_pitch(nx, fold_na(ny, nx));
}

}  // namespace fftamd
