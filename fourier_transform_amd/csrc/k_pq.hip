// C2C rows of length n = P * Q with P in {3, 5, 7, 9, 15, 25} and Q a power of
// two, 8192 < n <= 16384 (one Q per P), in one kernel with the data in
// registers.  This
// is the four-step split inside a workgroup ("High Performance Fourier
// Transforms on GPUs with GLSL", section 2.3 names mixed radices as the way
// beyond powers of two): element j = p + P q of a row,
//   1. the P interleaved sub-rows x[p + P q] (q < Q) are transformed with the
//      power-of-two Stockham stages, as P lines of the row kernel;
//   2. Y_p[k] is multiplied by W_n^{p k};
//   3. through LDS, a P-point DFT over p for every k gives X[k + Q k'].
// The P-point DFTs pair inputs p and P - p with cosine/sine constants written
// to 25 digits (rounded once).
#include "kernels.hpp"

namespace fftamd {

namespace {
// cos and sin of 2 pi q / P, q = 0 .. (P-1)/2 (a switch, so that device code
// needs no constant table in memory even where a loop is not unrolled)
template <int P>
__device__ __forceinline__ float odd_cos(int q);
template <int P>
__device__ __forceinline__ float odd_sin(int q);
template <>
__device__ __forceinline__ float odd_cos<3>(int q) {
  switch (q) {
    case 0: return 1.0f;
    case 1: return -0.5000000000000000000000000f;
    default: return 0.f;
  }
}
template <>
__device__ __forceinline__ float odd_sin<3>(int q) {
  switch (q) {
    case 0: return 0.0f;
    case 1: return 0.8660254037844386467637232f;
    default: return 0.f;
  }
}
template <>
__device__ __forceinline__ float odd_cos<5>(int q) {
  switch (q) {
    case 0: return 1.0f;
    case 1: return 0.3090169943749474241022934f;
    case 2: return -0.8090169943749474241022934f;
    default: return 0.f;
  }
}
template <>
__device__ __forceinline__ float odd_sin<5>(int q) {
  switch (q) {
    case 0: return 0.0f;
    case 1: return 0.9510565162951535721164393f;
    case 2: return 0.5877852522924731291687060f;
    default: return 0.f;
  }
}
template <>
__device__ __forceinline__ float odd_cos<7>(int q) {
  switch (q) {
    case 0: return 1.0f;
    case 1: return 0.6234898018587335305250049f;
    case 2: return -0.2225209339563144042889026f;
    case 3: return -0.9009688679024191262361023f;
    default: return 0.f;
  }
}
template <>
__device__ __forceinline__ float odd_sin<7>(int q) {
  switch (q) {
    case 0: return 0.0f;
    case 1: return 0.7818314824680298087084445f;
    case 2: return 0.9749279121818236070181317f;
    case 3: return 0.4338837391175581204757683f;
    default: return 0.f;
  }
}
template <>
__device__ __forceinline__ float odd_cos<9>(int q) {
  switch (q) {
    case 0: return 1.0f;
    case 1: return 0.7660444431189780352023927f;
    case 2: return 0.1736481776669303488517166f;
    case 3: return -0.5000000000000000000000000f;
    case 4: return -0.9396926207859083840541093f;
    default: return 0.f;
  }
}
template <>
__device__ __forceinline__ float odd_sin<9>(int q) {
  switch (q) {
    case 0: return 0.0f;
    case 1: return 0.6427876096865393263226434f;
    case 2: return 0.9848077530122080593667430f;
    case 3: return 0.8660254037844386467637232f;
    case 4: return 0.3420201433256687330440996f;
    default: return 0.f;
  }
}
template <>
__device__ __forceinline__ float odd_cos<15>(int q) {
  switch (q) {
    case 0: return 1.0f;
    case 1: return 0.9135454576426008955021276f;
    case 2: return 0.6691306063588582138262733f;
    case 3: return 0.3090169943749474241022934f;
    case 4: return -0.1045284632676534713998342f;
    case 5: return -0.5000000000000000000000000f;
    case 6: return -0.8090169943749474241022934f;
    case 7: return -0.9781476007338056379285667f;
    default: return 0.f;
  }
}
template <>
__device__ __forceinline__ float odd_sin<15>(int q) {
  switch (q) {
    case 0: return 0.0f;
    case 1: return 0.4067366430758002077539860f;
    case 2: return 0.7431448254773942350146970f;
    case 3: return 0.9510565162951535721164393f;
    case 4: return 0.9945218953682733369226919f;
    case 5: return 0.8660254037844386467637232f;
    case 6: return 0.5877852522924731291687060f;
    case 7: return 0.2079116908177593371017423f;
    default: return 0.f;
  }
}
template <>
__device__ __forceinline__ float odd_cos<25>(int q) {
  switch (q) {
    case 0: return 1.0f;
    case 1: return 0.9685831611286311194901684f;
    case 2: return 0.8763066800438635873081159f;
    case 3: return 0.7289686274214115231467303f;
    case 4: return 0.5358267949789966182713088f;
    case 5: return 0.3090169943749474241022934f;
    case 6: return 0.0627905195293133760761782f;
    case 7: return -0.1873813145857246305425507f;
    case 8: return -0.4257792915650726488625024f;
    case 9: return -0.6374239897486897101767128f;
    case 10: return -0.8090169943749474241022934f;
    case 11: return -0.9297764858882514036609426f;
    case 12: return -0.9921147013144778310497930f;
    default: return 0.f;
  }
}
template <>
__device__ __forceinline__ float odd_sin<25>(int q) {
  switch (q) {
    case 0: return 0.0f;
    case 1: return 0.2486898871648547882422837f;
    case 2: return 0.4817536741017152749871915f;
    case 3: return 0.6845471059286886737322834f;
    case 4: return 0.8443279255020150785485581f;
    case 5: return 0.9510565162951535721164393f;
    case 6: return 0.9980267284282715619523368f;
    case 7: return 0.9822872507286886810856417f;
    case 8: return 0.9048270524660195277136686f;
    case 9: return 0.7705132427757892308030096f;
    case 10: return 0.5877852522924731291687060f;
    case 11: return 0.3681245526846779591569471f;
    case 12: return 0.1253332335643042453731188f;
    default: return 0.f;
  }
}

// y_k = sum_p x_p e^{S 2 pi i pk/P} for odd P: y_0 = sum x,
// y_k = x_0 + a_k + S i b_k and y_{P-k} = x_0 + a_k - S i b_k with
// a_k = sum_j cos(2 pi jk/P)(x_j + x_{P-j}), b_k = sum_j sin(2 pi jk/P)(x_j - x_{P-j}).
template <int P, int S>
__device__ __forceinline__ void dft_odd(float2* x) {
  constexpr int H = (P - 1) / 2;
  float2 sp[H], sm[H];
  float2 y0 = x[0];
#pragma unroll
  for (int j = 1; j <= H; ++j) {
    sp[j - 1] = cadd(x[j], x[P - j]);
    sm[j - 1] = csub(x[j], x[P - j]);
    y0 = cadd(y0, sp[j - 1]);
  }
  float2 out[P];
  out[0] = y0;
#pragma unroll
  for (int k = 1; k <= H; ++k) {
    float2 a = x[0], b = make_float2(0.f, 0.f);
#pragma unroll
    for (int j = 1; j <= H; ++j) {
      const int e = (j * k) % P;
      const int q = e <= H ? e : P - e;  // cos/sin(2 pi e/P) from the first half-period
                                         // (e = 0 occurs for composite P)
      const float c = odd_cos<P>(q);
      const float s = e <= H ? odd_sin<P>(q) : -odd_sin<P>(q);
      a = make_float2(a.x + c * sp[j - 1].x, a.y + c * sp[j - 1].y);
      b = make_float2(b.x + s * sm[j - 1].x, b.y + s * sm[j - 1].y);
    }
    const float2 ib = mul_si<S>(b);
    out[k] = cadd(a, ib);
    out[P - k] = csub(a, ib);
  }
#pragma unroll
  for (int k = 0; k < P; ++k) x[k] = out[k];
}

// lines of length Q per workgroup: C rows of P lines each
constexpr int pq_rows(int q, int p) {
  const int t = pq_threads(q) * p;
  return t >= 256 ? 1 : 256 / t;
}
}  // namespace

template <int Q, int P, int S, int C>
__global__ __launch_bounds__(pq_threads(Q) * P * C) void k_c2c_pq(PqArgs a) {
  constexpr int E = pq_values(Q);
  constexpr int T = Q / E;
  constexpr int N = P * Q;
  constexpr int NT = C * P * T;
  constexpr bool WL = T <= 64 && (64 % T) == 0;  // each line inside one wavefront
  using L = RowLds<Q>;
  static_assert(row_lds_bytes(Q, C * P) <= kLdsBudgetBytes, "LDS budget");
  __shared__ float2 lds[L::size(C * P)];
  lds_poison(lds);

  const int tid = threadIdx.x;
  const int line = tid / T, u = tid - line * T;  // line = c P + p
  const int c = line / P, p = line - c * P;
  const int64_t row = (int64_t)blockIdx.x * C + c;
  const bool valid = row < a.rows;
  float2 v[E];
  if constexpr (P >= 7) {
    // Line p reads elements P apart, so a wavefront's loads would touch P *
    // 512 B.  Instead the group's C rows are loaded coalesced and put into
    // the line layout through LDS (element j of row cc: line cc P + j % P,
    // position j / P).  Per 512 MiB: 15360 801 -> 392 us, 12800 583 -> 434,
    // 14336 541 -> 400, 9216 501 -> 443; 10240 (P = 5) equal, 12288 (P = 3)
    // 403 -> 412, so those keep the direct loads.
    static_assert((C * N) % NT == 0 && (C * N) / NT == E, "one value per slot");
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint32_t e = (uint32_t)tid + (uint32_t)NT * i;
      const uint32_t cc = e / N, j = e - cc * N;
      const int64_t r = (int64_t)blockIdx.x * C + cc;
      float2 x = make_float2(0.f, 0.f);
      if (r < a.rows) {
        x = gload_nt(a.in + r * N, j);
        if (a.shift && (j & 1)) x = negate_bits(x);  // (-1)^j
      }
      lds[L::at((int)(cc * P + j % P), (int)(j / P))] = x;
    }
    lds_barrier();
    static_for<0, E>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      v[m] = lds[L::template at_k<T * m>(line, u)];
    });
    lds_barrier();  // stage 0 writes LDS again
  } else if (valid) {
    const float2* src = a.in + row * N;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const uint32_t j = (uint32_t)(p + P * (u + T * m));
      v[m] = gload_nt(src, j);
      // shift: (-1)^j, j = p + P q has the parity of p + q (P odd)
      if (a.shift && ((p + u + T * m) & 1)) v[m] = negate_bits(v[m]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) v[m] = make_float2(0.f, 0.f);
  }
  run_stages<Q, E, S, WL, L, false>(v, lds, a.tw, u, line);
  // W_n^{p k}, k = u + T m
#pragma unroll
  for (int m = 0; m < E; ++m) v[m] = apply_tw<S>(v[m], gload(a.wn, (uint32_t)(p * (u + T * m))));
  lds_barrier();  // the last stage's LDS reads precede these writes
  static_for<0, E>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    lds[L::template at_k<T * m>(line, u)] = v[m];
  });
  lds_barrier();
  // P-point DFTs over p for every (row c, k): outputs k + Q k'
  for (int it = tid; it < C * Q; it += NT) {
    const int cc = it / Q, k = it - cc * Q;
    const int64_t r = (int64_t)blockIdx.x * C + cc;
    float2 y[P];
#pragma unroll
    for (int q = 0; q < P; ++q) y[q] = lds[L::at(cc * P + q, k)];
    dft_odd<P, S>(y);
    if (r < a.rows) {
      float2* dst = a.out + r * N;
#pragma unroll
      for (int q = 0; q < P; ++q) gstore_nt(dst, (uint32_t)(k + Q * q), y[q]);
    }
  }
}

namespace {
template <int P, int S>
struct PqOp {
  template <int Q>
  struct At {
    static hipError_t run(const PqArgs& a, hipStream_t st) {
      if constexpr (P * Q > kMaxPqLength || P * Q < kMinPqLength) {
        return hipErrorInvalidValue;
      } else {
        constexpr int C = pq_rows(Q, P);
        uint32_t grid;
        hipError_t e = grid_of(a.rows, C, &grid);
        if (e != hipSuccess) return e;
        FFTAMD_LAUNCH((k_c2c_pq<Q, P, S, C>), dim3(grid), dim3(pq_threads(Q) * P * C), 0, st, a);
        return hipGetLastError();
      }
    }
  };
};
template <int S>
hipError_t launch_pq_sign(int q, int p, const PqArgs& a, hipStream_t st) {
  switch (p) {
    case 3: return dispatch_pow2<PqOp<3, S>::template At, 4096, 4096>(q, a, st);
    case 5: return dispatch_pow2<PqOp<5, S>::template At, 2048, 2048>(q, a, st);
    case 7: return dispatch_pow2<PqOp<7, S>::template At, 2048, 2048>(q, a, st);
    case 9: return dispatch_pow2<PqOp<9, S>::template At, 1024, 1024>(q, a, st);
    case 15: return dispatch_pow2<PqOp<15, S>::template At, 1024, 1024>(q, a, st);
    case 25: return dispatch_pow2<PqOp<25, S>::template At, 512, 512>(q, a, st);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_pq(int q, int p, int sign, const PqArgs& a, hipStream_t st) {
  if (a.rows < 1) return hipErrorInvalidValue;
  return sign < 0 ? launch_pq_sign<-1>(q, p, a, st) : launch_pq_sign<1>(q, p, a, st);
}

}  // namespace fftamd
