// The chirp transform above m = 16384 in three passes over HBM.
//
// Bluestein's method needs the forward transform of the chirped row, a
// product with the transform of the chirp, and the inverse transform of that
// product; m = n1 * n2 points, each transform a four-step split.  The
// forward transform's second factor (n1-point transforms along the rows k2
// of pass 1's block layout) produces bins k = k2 + n2*k1 row by row, and the
// inverse transform, split the same way with k = k2 + n2*k1 and output index
// j = j1 + n1*j2,
//   z[j1 + n1 j2] = sum_k2 W_m^{-j1 k2} W_n2^{-j2 k2} sum_k1 Z[k2 + n2 k1] W_n1^{-j1 k1},
// starts with n1-point transforms over k1 along the same rows.  So one row
// pass (k_chirp_mid) takes a row k2 through the forward n1-point transform,
// the product with the chirp's transform, the inverse n1-point transform
// and the factor W_m^{-j1 k2}; a column pass (k_chirp_out) finishes with the
// n2-point inverse transforms over k2 and the output chirp.  Against two
// full four-step transforms this saves one pass and the transposing store.
#include "kernels.hpp"

namespace fftamd {

// ---------------------------------------------------------------------------
// rows k2 of the block layout (BC columns per pass-1 workgroup): forward
// N1-point transform, times bt[k2*N1 + k1] (the chirp's transform at bin
// k2 + n2*k1, divided by m), inverse N1-point transform, times W_m^{-j1*k2};
// row k2 stored contiguously (n1 values) in out
// ---------------------------------------------------------------------------
template <int N1, int BC>
__global__ __launch_bounds__(tile_lines(N1, true) * (N1 / tile_e(N1, true))) void k_chirp_mid(FourStepArgs a) {
  constexpr int E = tile_e(N1, true);
  constexpr bool SPLIT = tile_split(N1, true);
  constexpr int C = tile_lines(N1, true);
  constexpr int T = N1 / E;
  constexpr int NT = C * T;
  constexpr bool WL = T <= 64;
  constexpr int FP = E + 1;
  using L = RowLds<N1, SPLIT, E>;
  constexpr int LB = L::size(C) * sizeof(lds_elem_t<SPLIT>) + C * FP * sizeof(float2);
  static_assert(LB <= kLdsBudgetBytes, "LDS budget");
  // stage-1 twiddles from an LDS copy when it fits (as in k_fs_rows), for the
  // forward and the inverse stages
  constexpr int TW1 = fs_tw1_elems<N1, E>();
  constexpr bool LTW = sched_stages(N1, E) >= 2 && LB + TW1 * sizeof(float2) <= kLdsBudgetBytes;
  constexpr int TQ = LTW ? (TW1 + NT - 1) / NT : 1;
  __shared__ lds_elem_t<SPLIT> lds[L::size(C)];
  __shared__ float2 ftab[C * FP];
  __shared__ float2 twl[LTW ? TW1 : 1];
  lds_poison(lds, ftab, twl);

  const int tid = threadIdx.x;
  const int line = tid / T, u = tid % T;
  const int64_t n2 = a.n2;
  const int64_t g0 = (int64_t)xcd_grouped_block(blockIdx.x, gridDim.x) * C;  // whole groups
  const int64_t b = g0 / n2;
  const uint32_t k20 = (uint32_t)(g0 - b * n2);
  const uint32_t k2 = k20 + (uint32_t)line;
  // W_m^{k2*j1} with j1 = u + T*m as W_m^{k2*u} * W_m^{k2*T*m}: a factor per
  // thread and a C x E table per workgroup (as in k_fs_cols), both from the
  // two-level table; k2*j1 < m
  const uint32_t mask = (1u << a.bits) - 1u;
  constexpr int FQ = (C * E + NT - 1) / NT;
  float2 fh[FQ], fl[FQ];
  float2 tq[TQ];
  if constexpr (LTW) fs_fetch_tw1<N1, E, NT, TQ>(tq, a.tw, tid);
#pragma unroll
  for (int i = 0; i < FQ; ++i) {
    const int q = tid + NT * i;
    if (q < C * E) {
      const uint32_t e = (k20 + (uint32_t)(q / E)) * (uint32_t)(T * (q % E));
      fh[i] = gload(a.thi, e >> a.bits);
      fl[i] = gload(a.tlo, e & mask);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float2 v[E];
  {
    const float2* src = a.in + g0 * N1;
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = gload_nt(src, fs_block_index<C, BC>((uint32_t)line, (uint32_t)(u + T * m), N1));
  }
  // bins k = k2 + n2*k1, k1 = u + T*m are multiplied by the chirp's transform
  // after the forward stages.  With 16 values per thread its loads and those
  // of W_m^{k2*u} are issued here, behind the row's loads, so the workgroup
  // waits for memory once; with 64 values per thread the VGPR budget keeps
  // them after the stages (in groups of 8).
  constexpr bool EARLY = E <= 16;
  const float2* bt = a.pre + (int64_t)k20 * N1;  // uniform base, 32-bit offsets
  const uint32_t bo = (uint32_t)line * N1 + (uint32_t)u;
  const uint32_t eu = k2 * (uint32_t)u;
  float2 bv[EARLY ? E : 1];
  float2 uh, ul;
  if constexpr (EARLY) {
#pragma unroll
    for (int m = 0; m < E; ++m) bv[m] = gload(bt, bo + (uint32_t)(T * m));
    uh = gload(a.thi, eu >> a.bits);
    ul = gload(a.tlo, eu & mask);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < FQ; ++i) {
    const int q = tid + NT * i;
    if (q < C * E) ftab[(q / E) * FP + q % E] = cmul(fh[i], fl[i]);
  }
  const TwLdsStage<1> tws{a.tw, twl, (uint32_t)sched_tw_off(N1, E, 1)};
  const auto tw = [&]() {
    if constexpr (LTW) {
      return tws;
    } else {
      return a.tw;
    }
  }();
  if constexpr (LTW) {
    fs_store_tw1<N1, E, NT, TQ>(twl, tq, tid);
    lds_barrier();  // the stage exchanges may be wave-local: publish the copy here
  }
  run_stages<N1, E, -1, WL, L, SPLIT>(v, lds, tw, u, line);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < E; ++m) {
    if constexpr (EARLY) {
      v[m] = cmul(v[m], bv[m]);
    } else {
      v[m] = cmul(v[m], gload(bt, bo + (uint32_t)(T * m)));
      if ((m & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
  }
  lds_barrier();  // the forward stages' last reads precede the inverse stages' writes; publishes ftab
  run_stages<N1, E, 1, WL, L, SPLIT>(v, lds, tw, u, line);
  if constexpr (!EARLY) {  // fetched here: live across the stages it would spill
    uh = gload(a.thi, eu >> a.bits);
    ul = gload(a.tlo, eu & mask);
  }
  const float2 wu = cmul(uh, ul);
  float2* dst = a.out + (g0 + line) * N1;
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const float2 w = cmul(wu, ftab[line * FP + m]);
    gstore_nt(dst, (uint32_t)(u + T * m), apply_tw<1>(v[m], w));
    if constexpr (E > 16) {
      if ((m & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------------------
// columns j1 of [batch][n2][n1] (rows k2): inverse N2-point transforms over
// k2, output j = j1 + n1*j2 kept for j < out_len, times post[j], stored to
// row b of out (out_stride apart)
// ---------------------------------------------------------------------------
template <int N2>
__global__ __launch_bounds__(tile_lines(N2, false) * (N2 / tile_e(N2, false))) void k_chirp_out(FourStepArgs a) {
  constexpr int E = tile_e(N2, false);
  constexpr bool SPLIT = tile_split(N2, false);
  constexpr int C = tile_lines(N2, false);
  constexpr int T = N2 / E;
  using L = ColLds<N2, C, SPLIT>;
  static_assert(L::size(C) * sizeof(lds_elem_t<SPLIT>) <= kLdsBudgetBytes, "LDS budget");
  __shared__ lds_elem_t<SPLIT> lds[L::size(C)];
  lds_poison(lds);

  const int tid = threadIdx.x;
  const int line = tid % C, u = tid / C;
  const int64_t g0 = (int64_t)xcd_grouped_block(blockIdx.x, gridDim.x) * C;  // whole groups
  const uint32_t n1 = (uint32_t)a.n1;
  const int64_t b = g0 / n1;
  const uint32_t c0 = (uint32_t)(g0 - b * n1);
  const uint32_t off = (uint32_t)line + (uint32_t)u * n1;
  const uint32_t step = (uint32_t)T * n1;
  float2 v[E];
  {
    const float2* src = a.in + b * (int64_t)n1 * N2 + c0;
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = gload_nt(src, off + step * m);
  }
  run_stages<N2, E, 1, false, L, SPLIT>(v, lds, a.tw, u, line);
  __builtin_amdgcn_sched_barrier(0);  // keep the post loads below the stages (VGPR budget)
  float2* dst = a.out + b * a.out_stride + c0;
  // The store offsets are recomputed from an opaque copy of off: reusing the
  // load offsets kept 64 of them live across the stages (spilled).
  uint32_t off2 = off;
  asm volatile("" : "+v"(off2));
  // Outputs j >= out_len are dropped.  With 64 values per thread a branch per
  // store costs many VGPRs spilled, so those tiles write the dropped outputs
  // to a.sink instead (a scratch row that nothing reads any more).
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const uint32_t o = off2 + step * m;
    const uint32_t j = c0 + o;
    const bool keep = j < (uint32_t)a.out_len;
    if constexpr (E > 16) {
      float2* q = keep ? dst + o : a.sink + tid;
      gstore_nt(q, 0u, cmul(v[m], gload(a.post, keep ? j : 0u)));
      if ((m & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    } else if (keep) {
      gstore_nt(dst, o, cmul(v[m], gload(a.post, j)));
    }
  }
}

namespace {
struct ChirpMidOp {
  template <int N1>
  struct At {
    template <int BC>
    static hipError_t go(const FourStepArgs& a, hipStream_t st) {
      constexpr int C = tile_lines(N1, true);
      if ((a.batch * a.n2) % C != 0) return hipErrorInvalidValue;  // whole groups
      uint32_t grid;
      hipError_t e = grid_of(a.batch * a.n2, C, &grid);
      if (e != hipSuccess) return e;
      FFTAMD_LAUNCH((k_chirp_mid<N1, BC>), dim3(grid), dim3(C * (N1 / tile_e(N1, true))), 0, st, a);
      return hipGetLastError();
    }
    static hipError_t run(const FourStepArgs& a, hipStream_t st) {
      // pass 1 (k_fs_cols over n2 points) wrote blocks tile_lines(n2) columns wide
      if (a.n2 == N1) return go<tile_lines(N1, false)>(a, st);
      if (a.n2 == 2 * N1) return go<tile_lines(2 * N1, false)>(a, st);
      return hipErrorInvalidValue;
    }
  };
};
struct ChirpOutOp {
  template <int N2>
  struct At {
    static hipError_t run(const FourStepArgs& a, hipStream_t st) {
      constexpr int C = tile_lines(N2, false);
      if ((a.batch * a.n1) % C != 0) return hipErrorInvalidValue;  // whole groups
      uint32_t grid;
      hipError_t e = grid_of(a.batch * a.n1, C, &grid);
      if (e != hipSuccess) return e;
      FFTAMD_LAUNCH((k_chirp_out<N2>), dim3(grid), dim3(C * (N2 / tile_e(N2, false))), 0, st, a);
      return hipGetLastError();
    }
  };
};
// the split of m = 2^15 .. 2^23: n1 = 2^7 .. 2^11, n2 = 2^8 .. 2^12
constexpr int kChirpRowsMin = 128, kChirpRowsMax = 2048;
constexpr int kChirpColsMin = 256, kChirpColsMax = 4096;
}  // namespace

hipError_t launch_chirp_mid(int n1, const FourStepArgs& a, hipStream_t st) {
  if (!a.pre) return hipErrorInvalidValue;
  return dispatch_pow2<ChirpMidOp::At, kChirpRowsMin, kChirpRowsMax>(n1, a, st);
}
hipError_t launch_chirp_out(int n2, const FourStepArgs& a, hipStream_t st) {
  if (!a.post || !a.sink || a.out_len < 1 || (int64_t)a.out_len > (int64_t)a.n1 * a.n2) return hipErrorInvalidValue;
  return dispatch_pow2<ChirpOutOp::At, kChirpColsMin, kChirpColsMax>(n2, a, st);
}

}  // namespace fftamd
