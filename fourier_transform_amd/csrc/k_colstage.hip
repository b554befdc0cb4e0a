// Column-stage kernel and its launcher: the two steps of the column transform
// of tall 2D images (see ColStageArgs in launch.hpp).  Each workgroup takes up
// to 64 adjacent columns of a short sub-column, so every HBM access is a run
// of up to 512 B, and the tile (about 32 KiB) leaves room for several
// workgroups per CU.
#include "kernels.hpp"

namespace fftamd {

template <int L, int S, bool TWID>
__global__ __launch_bounds__(colstage_lines(L) * (L / colstage_values(L))) void k_col_stage(ColStageArgs a) {
  constexpr int E = colstage_values(L);
  constexpr int C = colstage_lines(L);
  constexpr int T = L / E;
  using L_ = ColLds<L, C, false>;
  static_assert(L_::size(C) * sizeof(float2) <= kLdsBudgetBytes, "LDS budget");
  __shared__ float2 lds[L_::size(C)];
  lds_poison(lds);

  const int tid = threadIdx.x;
  const int line = tid % C, u = tid / C;
  const int64_t c = (int64_t)blockIdx.x * C + line;
  const bool valid = c < a.nlines;
  const uint32_t q = (uint32_t)(c >> a.log2nx), r = (uint32_t)c & (a.nx - 1);
  const int64_t img = (int64_t)blockIdx.y * a.image_stride;
  const float2* src = a.in + img + (int64_t)q * a.a_in + r;
  float2* dst = a.out + img + (int64_t)q * a.a_out + r;
  float2 v[E];
  if (valid) {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = gload_nt(src, (uint32_t)(u + T * m) * a.s_in);
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = make_float2(0.f, 0.f);
  }
  run_stages<L, E, S, false, L_, false>(v, lds, a.tw, u, line);
  if (valid) {
#pragma unroll
    for (int m = 0; m < E; ++m) {
      float2 y = v[m];
      if constexpr (TWID) y = apply_tw<S>(y, gload(a.wt, q * (uint32_t)(u + T * m)));
      gstore(dst, (uint32_t)(u + T * m) * a.s_out, y);
    }
  }
}

namespace {
template <int S, bool TW>
struct ColStageOp {
  template <int L>
  struct At {
    static hipError_t run(const ColStageArgs& a, hipStream_t st) {
      constexpr int C = colstage_lines(L);
      uint32_t grid;
      hipError_t e = grid_of(a.nlines, C, &grid);
      if (e != hipSuccess) return e;
      if (a.images < 1 || a.images > 65535) return hipErrorInvalidConfiguration;
      FFTAMD_LAUNCH((k_col_stage<L, S, TW>), dim3(grid, a.images), dim3(C * (L / colstage_values(L))), 0, st, a);
      return hipGetLastError();
    }
  };
};
}  // namespace

// lengths used by the split of columns of 2048 .. 16384 rows (64 x 32 .. 64 x 256)
constexpr int kColStageMin = 16;
constexpr int kColStageMax = 256;

hipError_t launch_col_stage(int len, int sign, bool twiddle, const ColStageArgs& a, hipStream_t st) {
  if (sign < 0) {
    return twiddle ? dispatch_pow2<ColStageOp<-1, true>::At, kColStageMin, kColStageMax>(len, a, st)
                   : dispatch_pow2<ColStageOp<-1, false>::At, kColStageMin, kColStageMax>(len, a, st);
  }
  return twiddle ? dispatch_pow2<ColStageOp<1, true>::At, kColStageMin, kColStageMax>(len, a, st)
                 : dispatch_pow2<ColStageOp<1, false>::At, kColStageMin, kColStageMax>(len, a, st);
}

}  // namespace fftamd
