// Mixed-radix Stockham transform for C2C rows whose length has no prime
// factor above 7 (radices 2, 3, 4, 5, 7, 8).  The GLSL dissertation ("High
// Performance Fourier Transforms on GPUs with GLSL", section 2.3) names
// mixed radices as the way beyond powers of two; the stage itself is the
// natural-order Stockham step of the WGSL Fourier-stage source (turing-sphere
// fourier.ts, stockham()) with a radix that changes from stage to stage:
// butterfly b reads b + r*m (m = n/R), twiddles input r by W_{ns R}^{r j}
// (j = b mod ns, ns = product of the earlier radices), runs an R-point DFT
// and writes output q to (b - j) R + j + q ns.
//
// One kernel handles every such length: the schedule is plan data, each
// thread holds up to 2 butterflies of at most 8 values in registers, and the line lives in LDS between stages (read, barrier,
// compute, write, barrier).  The first stage reads HBM directly and the last
// one writes it, both coalesced (consecutive butterflies, consecutive
// addresses).
#include "kernels.hpp"

namespace fftamd {

namespace {
// R-point DFT for an odd prime R by pairing inputs j and R - j:
// y_0 = sum x, y_k = x_0 + a_k + S i b_k, y_{R-k} = x_0 + a_k - S i b_k with
// a_k = sum_j cos(2 pi jk/R)(x_j + x_{R-j}), b_k = sum_j sin(2 pi jk/R)(x_j - x_{R-j}),
// j, k = 1 .. (R-1)/2.  Constants written to 25 digits, rounded once.
template <int R>
__device__ __forceinline__ float cosq(int k) {
  if constexpr (R == 3) {
    return -0.5f;
  } else if constexpr (R == 5) {
    return k == 1 ? 0.3090169943749474241022934f : -0.8090169943749474241022934f;
  } else {
    return k == 1 ? 0.6234898018587335305250049f
                  : (k == 2 ? -0.2225209339563144042889026f : -0.9009688679024191262361023f);
  }
}
template <int R>
__device__ __forceinline__ float sinq(int k) {
  if constexpr (R == 3) {
    return 0.8660254037844386467637232f;
  } else if constexpr (R == 5) {
    return k == 1 ? 0.9510565162951535721164393f : 0.5877852522924731291687060f;
  } else {
    return k == 1 ? 0.7818314824680298087084445f
                  : (k == 2 ? 0.9749279121818236070181317f : 0.4338837391175581204757683f);
  }
}
template <int R, int S>
__device__ __forceinline__ void dft_prime(float2* x) {
  constexpr int H = (R - 1) / 2;
  float2 sp[H], sm[H];
  float2 y0 = x[0];
#pragma unroll
  for (int j = 1; j <= H; ++j) {
    sp[j - 1] = cadd(x[j], x[R - j]);
    sm[j - 1] = csub(x[j], x[R - j]);
    y0 = cadd(y0, sp[j - 1]);
  }
  float2 out[R];
  out[0] = y0;
#pragma unroll
  for (int k = 1; k <= H; ++k) {
    float2 a = x[0], b = make_float2(0.f, 0.f);
#pragma unroll
    for (int j = 1; j <= H; ++j) {
      const int e = (j * k) % R;  // cos/sin(2 pi jk/R) from the first half-period
      const int q = e <= H ? e : R - e;
      const float c = cosq<R>(q), s = e <= H ? sinq<R>(q) : -sinq<R>(q);
      a = make_float2(a.x + c * sp[j - 1].x, a.y + c * sp[j - 1].y);
      b = make_float2(b.x + s * sm[j - 1].x, b.y + s * sm[j - 1].y);
    }
    const float2 ib = mul_si<S>(b);  // S i b
    out[k] = cadd(a, ib);
    out[R - k] = csub(a, ib);
  }
#pragma unroll
  for (int k = 0; k < R; ++k) x[k] = out[k];
}

template <int S>
__device__ __forceinline__ void dft_any(int R, float2* x) {
  switch (R) {
    case 2: dft<2, S>(x); break;
    case 3: dft_prime<3, S>(x); break;
    case 4: dft<4, S>(x); break;
    case 5: dft_prime<5, S>(x); break;
    case 7: dft_prime<7, S>(x); break;
    default: dft<8, S>(x); break;
  }
}

__host__ __device__ __forceinline__ uint32_t mixed_pad(uint32_t i) { return i + (i >> 5); }
}  // namespace

// KB = 2 butterflies of at most 8 values per thread and stage, up to 1024
// threads (so at most 128 VGPRs)
template <int S, int KB>
__global__ __launch_bounds__(1024) void k_mixed(MixedArgs a) {
  extern __shared__ float4 smem4[];
  float2* smem = reinterpret_cast<float2*>(smem4);
  const int tpl = a.tpl;
  const int tid = threadIdx.x;
  const int line = tid / tpl, t = tid - line * tpl;
  const int64_t row = (int64_t)blockIdx.x * a.lines + line;
  const bool valid = row < a.rows;
  const uint32_t n = (uint32_t)a.n;
  float2* L = smem + (size_t)line * (mixed_pad(n) + 1);
  const float2* src = a.in + row * n;
  float2* dst = a.out + row * n;

  float2 x[KB][8];
  for (int s = 0; s < a.nstages; ++s) {
    const int R = a.radix[s];
    const uint32_t ns = (uint32_t)a.ns[s], m = (uint32_t)a.m[s];
    // gather the inputs of this thread's butterflies: b + r*m
    if (s == 0) {
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const uint32_t b = (uint32_t)(t + tpl * i);
        if (valid && b < m) {
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            if (r < R) {
              float2 v = gload_nt(src, b + r * m);
              if (a.pre) v = cmul(v, gload(a.pre, b + r * m));
              x[i][r] = v;
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const uint32_t b = (uint32_t)(t + tpl * i);
        if (b < m) {
#pragma unroll
          for (int r = 0; r < 8; ++r)
            if (r < R) x[i][r] = L[mixed_pad(b + r * m)];
        }
      }
      lds_barrier();  // every read of this stage precedes its writes
    }
    // twiddles and the R-point DFTs
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const uint32_t b = (uint32_t)(t + tpl * i);
      if (b < m) {
        if (s > 0) {
          const uint32_t j = b - __umulhi(b, a.ns_magic[s]) * ns;
          const float2* tw = a.tw + a.twoff[s] + j;
#pragma unroll
          for (int r = 1; r < 8; ++r)
            if (r < R) x[i][r] = apply_tw<S>(x[i][r], tw[(r - 1) * ns]);
        }
        dft_any<S>(R, x[i]);
      }
    }
    // scatter the outputs: (b - j) R + j + q ns
    if (s + 1 < a.nstages) {
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const uint32_t b = (uint32_t)(t + tpl * i);
        if (b < m) {
          const uint32_t j = ns == 1 ? 0u : b - __umulhi(b, a.ns_magic[s]) * ns;
          const uint32_t base = (b - j) * (uint32_t)R + j;
#pragma unroll
          for (int r = 0; r < 8; ++r)
            if (r < R) L[mixed_pad(base + r * ns)] = x[i][r];
        }
      }
      lds_barrier();
    } else if (valid) {
      // last stage: ns = m and j = b, so output q of butterfly b is b + q m
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const uint32_t b = (uint32_t)(t + tpl * i);
        if (b < m) {
#pragma unroll
          for (int r = 0; r < 8; ++r)
            if (r < R) gstore_nt(dst, b + r * ns, x[i][r]);
        }
      }
    }
  }
}

hipError_t launch_mixed(int sign, const MixedArgs& a, hipStream_t st) {
  if (a.n < 2 || a.n > kMaxMixedLength || a.nstages < 1 || a.nstages > kMixedMaxStages || a.tpl < 1 ||
      a.lines < 1 || a.tpl * a.lines > 1024 || a.rows < 1 || a.kb != kMixedButterflies)
    return hipErrorInvalidValue;
  for (int s = 0; s < a.nstages; ++s)  // every butterfly of every stage has a thread
    if ((int64_t)a.tpl * a.kb < a.m[s]) return hipErrorInvalidValue;
  uint32_t grid;
  hipError_t e = grid_of(a.rows, a.lines, &grid);
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)a.lines * (mixed_pad((uint32_t)a.n) + 1) * sizeof(float2);
  if (lds > (size_t)kLdsBudgetBytes) return hipErrorInvalidValue;
  const dim3 block((uint32_t)(a.tpl * a.lines));
  if (sign < 0)
    hipLaunchKernelGGL((k_mixed<-1, kMixedButterflies>), dim3(grid), block, lds, st, a);
  else
    hipLaunchKernelGGL((k_mixed<1, kMixedButterflies>), dim3(grid), block, lds, st, a);
  return hipGetLastError();
}

}  // namespace fftamd
