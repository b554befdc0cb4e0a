// 2D images of 4096, 8192 and 16384 rows in two passes over HBM.
//
// A 2D transform is the row transforms followed by the column transforms
// (Mota, section 2.7, Equation 19).  Here the column transform of length
// ny = NA * NB is split as in the four-step method (named in "Fast Fourier
// Transform on CPU and GPU", Working Progress, for transforms that do not fit
// on chip): with row index y = yb + NB*ya and bin k = ka + NA*kb,
//   X[ka + NA*kb] = sum_yb W_NB^{yb*kb} W_ny^{yb*ka} sum_ya x[yb + NB*ya] W_NA^{ya*ka}
// (W_L = e^{sign 2 pi i/L}).  Row transforms along x commute with all of it.
//
// Pass 1 (k_rows_fold): one workgroup per (image, yb) holds the NA rows
// yb + NB*ya in registers, transforms each along x (Stockham stages, split
// LDS exchange), then exchanges once more so that every thread holds all NA
// rows at a few columns, runs the NA-point DFT across the rows, multiplies
// output ka by W_ny^{yb*ka} and stores it as row ka of group yb of the
// scratch: the NA rows a workgroup writes are adjacent.
//
// Pass 2 (k_fold_cols): for each ka, NB-point transforms of 16-column tiles
// over row ka of every scratch group (yb = 0 .. NB-1), stored to rows
// ka + NA*kb of the output, which hold bin ka + NA*kb: the natural order.
// Both sides are runs of 16 x 8 B = 128 B.  Each scratch group of NA rows is
// followed by a little padding, so pass 2 reads with a stride that is not a
// power of two; its writes keep the output's power-of-two row pitch.
//
// Against rows + two column steps this moves each element through HBM twice
// instead of three times; against rows + a 4096-point column pass (whose
// tiles hold 8 columns: 64 B runs) it keeps 128 B runs on both sides.
#include "kernels.hpp"

namespace fftamd {

// ---------------------------------------------------------------------------
// pass 1: N = nx, NA rows per workgroup, EF values per thread
//
// Tiles of 64 values per thread (one workgroup holds the CU) are persistent,
// as in four-step pass 2: one wave of workgroups, each looping over (image,
// yb) tiles, half of them starting 13 us late (stagger_start).  Measured per
// launch: 8192 x 8192 277 -> 243-248 us (6 us late: 270, 9: 264, 18: 273;
// persistent without the stagger: 272), 16384 x 4096 265 -> 236-239 us.  The
// same loop in pass 2 was slower (269 -> 277 us).
// ---------------------------------------------------------------------------
template <int EF>
constexpr bool fold_rows_persistent() {
  return EF == kSplitValues;
}
template <int N, int NA, int EF, int S>
__global__ __launch_bounds__(NA * N / EF) void k_rows_fold(FoldArgs a) {
  constexpr int E = EF;
  constexpr int T = N / E;   // threads per row
  constexpr int MP = E / NA;  // columns per thread in the step across rows
  constexpr bool WL = T <= 64;
  using L = RowLds<N, true, E>;
  static_assert(L::size(NA) * sizeof(float) <= kLdsBudgetBytes, "LDS budget");
  static_assert(T % 2 == 0 && MP >= 1, "fold shape");
  constexpr int NT = NA * T;
  // stage 1 reads its twiddles from an LDS copy (as in the four-step passes)
  constexpr int TW1 = fs_tw1_elems<N, E>();
  constexpr bool LTW = sched_stages(N, E) >= 2 && L::size(NA) * sizeof(float) + TW1 * sizeof(float2) <= kLdsBudgetBytes;
  constexpr int TQ = LTW ? (TW1 + NT - 1) / NT : 1;
  __shared__ float lds[L::size(NA)];
  __shared__ float2 twl[LTW ? TW1 : 1];
  lds_poison(lds, twl);

  constexpr bool PERSIST = fold_rows_persistent<EF>();
  if constexpr (LTW && PERSIST) {  // the stage-1 twiddles once per workgroup
    float2 tq[TQ];
    fs_fetch_tw1<N, E, NT, TQ>(tq, a.tw, threadIdx.x);
    fs_store_tw1<N, E, NT, TQ>(twl, tq, threadIdx.x);
    lds_barrier();  // the stage exchanges may be wave-local: publish the copy here
  }
  if constexpr (PERSIST) stagger_start(a.stagger);
  const uint32_t nb = (uint32_t)(a.ny / NA);
  const uint32_t ntiles = (uint32_t)(a.images * nb);
  for (uint32_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
  // a per-tile opaque copy of the thread index: what derives from it is
  // recomputed per tile rather than kept live across the loop
  int tid = threadIdx.x;
  if constexpr (PERSIST) asm volatile("" : "+v"(tid));
  const int line = tid / T, u = tid % T;
  const int64_t img = (int64_t)(tile / nb);
  const uint32_t yb = tile - (uint32_t)img * nb;
  // the small loads first (see k_fs_cols): W_ny^{yb*ka}, one factor per
  // output row (yb*ka < ny), and the stage-1 twiddles
  float2 w[NA];
#pragma unroll
  for (int ka = 1; ka < NA; ++ka) w[ka] = gload(a.wy, yb * (uint32_t)ka);
  float2 tq[TQ];
  if constexpr (LTW && !PERSIST) fs_fetch_tw1<N, E, NT, TQ>(tq, a.tw, tid);
  __builtin_amdgcn_sched_barrier(0);
  // rows yb + nb*line of the image; 32-bit offsets from a uniform base
  const float2* src = a.in + (img * a.ny + yb) * N;
  const uint32_t off = (uint32_t)line * nb * N + (uint32_t)u;
  float2 v[E];
  static_for<0, E>([&](auto ic) {
    constexpr int m = load_slot<N, E>(decltype(ic)::value);
    v[m] = gload_nt(src + T * m, off);
  });
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (LTW && !PERSIST) {
    fs_store_tw1<N, E, NT, TQ>(twl, tq, tid);
    lds_barrier();  // the stage exchanges may be wave-local: publish the copy here
  }
  if (a.shift && ((yb + (uint32_t)u) & 1)) {  // (-1)^(y + x): nb and T are even
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = negate_bits(v[m]);
  }
  if constexpr (LTW) {
    const TwLdsStage<1> tws{a.tw, twl, (uint32_t)sched_tw_off(N, E, 1)};
    run_stages<N, E, S, WL, L, true>(v, lds, tws, u, line);
  } else {
    run_stages<N, E, S, WL, L, true>(v, lds, a.tw, u, line);
  }

  // Across rows: thread (line, u) takes columns u + T*(line*MP + i), i < MP,
  // of every row; v[ya*MP + i] receives row ya.  Real parts, then imaginary.
  lds_barrier();
  const int i0 = u + T * MP * line;
  static_for<0, E>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    lds[L::template at_k<T * m>(line, u)] = v[m].x;
  });
  lds_barrier();
  static_for<0, NA>([&](auto yc) {
    constexpr int ya = decltype(yc)::value;
    static_for<0, MP>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      v[ya * MP + i].x = lds[L::template at_k<T * i>(ya, i0)];
    });
  });
  lds_barrier();
  int u2 = u, line2 = line, i02 = i0;  // recompute addresses (see run_stage)
  asm volatile("" : "+v"(u2), "+v"(line2), "+v"(i02));
  static_for<0, E>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    lds[L::template at_k<T * m>(line2, u2)] = v[m].y;
  });
  lds_barrier();
  static_for<0, NA>([&](auto yc) {
    constexpr int ya = decltype(yc)::value;
    static_for<0, MP>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      v[ya * MP + i].y = lds[L::template at_k<T * i>(ya, i02)];
    });
  });

  // scratch: group yb of image img, its NA rows adjacent.  Ordinary (not
  // streaming) stores, so that pass 2 finds part of it in the caches
  // (8192 x 8192: 549.6 -> 546.8 us, 16384 x 4096: 529.9 -> 523.1 us per exec)
  constexpr int64_t GP = fold_group_pitch(N, NA);
  float2* dst = a.out + (img * nb + yb) * GP;
#pragma unroll
  for (int i = 0; i < MP; ++i) {
    float2 x[NA];
#pragma unroll
    for (int ya = 0; ya < NA; ++ya) x[ya] = v[ya * MP + i];
    dft<NA, S>(x);
#pragma unroll
    for (int ka = 0; ka < NA; ++ka) {
      const float2 y = ka == 0 ? x[0] : apply_tw<S>(x[ka], w[ka]);
      gstore(dst, (uint32_t)(ka * N + i0 + T * i), y);
    }
  }
  if constexpr (!PERSIST) break;  // one tile per workgroup
  lds_barrier();  // the next tile's exchanges overwrite LDS
  }
}

// ---------------------------------------------------------------------------
// pass 2: NB-point column transforms over rows ka + NA*j, C adjacent columns
// per workgroup, E values per thread, split LDS exchange
// ---------------------------------------------------------------------------
template <int N, int C, int E, int S>
__global__ __launch_bounds__(C * N / E) void k_fold_cols(FoldArgs a) {
  constexpr int T = N / E;
  using L = ColLds<N, C, true>;
  static_assert(L::size(C) * sizeof(float) <= kLdsBudgetBytes, "LDS budget");
  constexpr int NT = C * T;
  constexpr int TW1 = fs_tw1_elems<N, E>();
  constexpr bool LTW = sched_stages(N, E) >= 2 && L::size(C) * sizeof(float) + TW1 * sizeof(float2) <= kLdsBudgetBytes;
  constexpr int TQ = LTW ? (TW1 + NT - 1) / NT : 1;
  __shared__ float lds[L::size(C)];
  __shared__ float2 twl[LTW ? TW1 : 1];
  lds_poison(lds, twl);

  const int tid = threadIdx.x;
  const int line = tid % C, u = tid / C;
  // column groups numbered (image, ka, x / C); nx is a multiple of C
  // Plain block order: the workgroups in flight together take adjacent
  // tiles across the whole chip, so each row's runs are read close together
  // in time (faster here than grouping adjacent tiles per XCD, which only
  // pays when runs are shorter than an L2 line).
  const int64_t g0 = (int64_t)blockIdx.x * C;
  const uint32_t nx = (uint32_t)a.nx;
  const int64_t vi = g0 / nx;
  const uint32_t x0 = (uint32_t)(g0 - vi * nx);
  const int na = (int)(a.ny / N);
  const int64_t img = vi / na;
  const int ka = (int)(vi - img * na);
  // input: the scratch, groups of na rows fold_group_pitch apart; output:
  // rows ka + na*j of the image
  const uint32_t gp = (uint32_t)fold_group_pitch(nx, na);
  const uint32_t pitch = (uint32_t)na * nx;
  float2 tq[TQ];
  if constexpr (LTW) fs_fetch_tw1<N, E, NT, TQ>(tq, a.tw2, tid);
  __builtin_amdgcn_sched_barrier(0);
  float2 v[E];
  {
    const float2* src = a.in + img * (a.ny / na) * gp + (int64_t)ka * nx + x0;
    const uint32_t off = (uint32_t)line + (uint32_t)u * gp;
    static_for<0, E>([&](auto ic) {
      constexpr int m = load_slot<N, E>(decltype(ic)::value);
      v[m] = gload_nt(src + (size_t)T * gp * m, off);
    });
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (LTW) {
    // stage 0's exchange barriers (workgroup-wide here) order these writes
    // before stage 1 reads them
    fs_store_tw1<N, E, NT, TQ>(twl, tq, tid);
    const TwLdsStage<1> tws{a.tw2, twl, (uint32_t)sched_tw_off(N, E, 1)};
    run_stages<N, E, S, false, L, true>(v, lds, tws, u, line);
  } else {
    run_stages<N, E, S, false, L, true>(v, lds, a.tw2, u, line);
  }
  const uint32_t off = (uint32_t)line + (uint32_t)u * pitch;
  const size_t step = (size_t)T * pitch;
  float2* dst = a.out + (img * a.ny + ka) * (int64_t)nx + x0;
#pragma unroll
  for (int m = 0; m < E; ++m) {
    gstore_nt(dst + step * m, off, v[m]);
    if constexpr (E > 16) {
      if ((m & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

namespace {
template <int NY, int NX, int S>
hipError_t run_fold(const FoldArgs& a, hipStream_t st) {
  constexpr int NA = fold_na(NY, NX);
  constexpr int NB = NY / NA;
  constexpr int E1 = fold_row_values(NX, NA);
  constexpr int C = fold_c(NB);
  constexpr int E2 = fold_col_values(NB, C);
  if (a.ny != NY || a.nx != NX || a.images < 1) return hipErrorInvalidValue;
  const int64_t g1 = a.images * NB;
  const int64_t g2 = a.images * NA * (NX / C);
  if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  FoldArgs p1 = a;
  p1.out = a.scratch;
  p1.stagger = 0;
  uint32_t grid1 = (uint32_t)g1;
  hipError_t e;
  if constexpr (fold_rows_persistent<E1>()) {
    uint32_t resident = 0;
    if ((e = resident_workgroups<k_rows_fold<NX, NA, E1, S>>(NA * NX / E1, &resident)) != hipSuccess) return e;
    if (grid1 > resident) grid1 = resident;
    if ((e = stagger_ticks(13.0, (uint32_t)g1, grid1, &p1.stagger)) != hipSuccess) return e;
  }
  FFTAMD_LAUNCH((k_rows_fold<NX, NA, E1, S>), dim3(grid1), dim3(NA * NX / E1), 0, st, p1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  FoldArgs p2 = a;
  p2.in = a.scratch;
  p2.stagger = 0;
  FFTAMD_LAUNCH((k_fold_cols<NB, C, E2, S>), dim3((uint32_t)g2), dim3(C * NB / E2), 0, st, p2);
  return hipGetLastError();
}

template <int NY, int S>
hipError_t fold_ny(const FoldArgs& a, hipStream_t st) {
  switch (a.nx) {
    case 512:
      return run_fold<NY, 512, S>(a, st);
    case 1024:
      return run_fold<NY, 1024, S>(a, st);
    case 2048:
      return run_fold<NY, 2048, S>(a, st);
    case 4096:
      return run_fold<NY, 4096, S>(a, st);
    case 8192:
      if constexpr (fold_fits(NY, 8192)) return run_fold<NY, 8192, S>(a, st);
      break;
    case 16384:
      if constexpr (fold_fits(NY, 16384)) return run_fold<NY, 16384, S>(a, st);
      break;
    default:
      break;
  }
  return hipErrorInvalidValue;
}

template <int S>
hipError_t fold_sign(const FoldArgs& a, hipStream_t st) {
  if (a.ny == 4096) return fold_ny<4096, S>(a, st);
  if (a.ny == 8192) return fold_ny<8192, S>(a, st);
  if (a.ny == 16384) return fold_ny<16384, S>(a, st);
  return hipErrorInvalidValue;
}
}  // namespace

// The two passes against the other forms, per exec on MI355X (512 MiB per
// exec where the image allows): against rows + two column steps (images of
// 8192 rows and more) 8192 x 8192 566 against 650 us, 16384 x 4096 551
// against 606, 8192 x 4096 295 against 303, 16384 x 2048 285 against 297,
// 8192 x 2048 and 16384 x 1024 115-120 against 150, 8192 x 1024 390 against
// 606, 8192 x 512 394 against 624, 16384 x 512 396 against 609; against rows
// + the 4096-point column pass (8 columns per workgroup, 64 B runs) 4096 x
// 4096 431 against 522, 4096 x 2048 405 against 511, 4096 x 1024 388 against
// 526, 4096 x 512 404 against 503, 4096 x 8192 548 against 574, 4096 x 16384
// 514 against 641.
bool fold_supported(int64_t ny, int64_t nx) { return fold_fits(ny, nx); }

hipError_t launch_fold_2d(int sign, const FoldArgs& a, hipStream_t st) {
  return sign < 0 ? fold_sign<-1>(a, st) : fold_sign<1>(a, st);
}

}  // namespace fftamd
