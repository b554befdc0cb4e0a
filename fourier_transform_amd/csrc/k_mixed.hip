// Mixed-radix Stockham transform for C2C rows whose length has no prime
// factor above 13 (radices 2..8, 10..16).  The GLSL dissertation ("High
// Performance Fourier Transforms on GPUs with GLSL", section 2.3) names
// mixed radices as the way beyond powers of two; the stage itself is the
// natural-order Stockham step of the WGSL Fourier-stage source (turing-sphere
// fourier.ts, stockham()) with a radix that changes from stage to stage:
// butterfly b reads b + r*m (m = n/R), twiddles input r by W_{ns R}^{r j}
// (j = b mod ns, ns = product of the earlier radices), runs an R-point DFT
// and writes output q to (b - j) R + j + q ns.
//
// One kernel handles every such length: the schedule is plan data, each
// thread holds one butterfly of up to 16 values or two of up to 8 (above 8192
// points two of up to 16) in registers, and the line lives in LDS between
// stages (read, barrier, compute, write, barrier).  The first stage reads HBM
// directly and the last one writes it (consecutive butterflies, consecutive
// addresses); lines of fewer than 128 threads, whose butterflies would read
// runs of a few elements, move the workgroup's block of rows through LDS in
// order instead.
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
  } else if constexpr (R == 7) {
    return k == 1 ? 0.6234898018587335305250049f
                  : (k == 2 ? -0.2225209339563144042889026f : -0.9009688679024191262361023f);
  } else if constexpr (R == 11) {
    switch (k) {
      case 1: return 0.8412535328311811688618116f;
      case 2: return 0.4154150130018864255292741f;
      case 3: return -0.1423148382732851404437927f;
      case 4: return -0.6548607339452850640569251f;
      default: return -0.9594929736144973898903681f;
    }
  } else {
    static_assert(R == 13, "radix");
    switch (k) {
      case 1: return 0.8854560256532098959003755f;
      case 2: return 0.5680647467311558025118076f;
      case 3: return 0.1205366802553230533490677f;
      case 4: return -0.3546048870425356259696379f;
      case 5: return -0.7485107481711010986346306f;
      default: return -0.9709418174260520271569823f;
    }
  }
}
template <int R>
__device__ __forceinline__ float sinq(int k) {
  if constexpr (R == 3) {
    return 0.8660254037844386467637232f;
  } else if constexpr (R == 5) {
    return k == 1 ? 0.9510565162951535721164393f : 0.5877852522924731291687060f;
  } else if constexpr (R == 7) {
    return k == 1 ? 0.7818314824680298087084445f
                  : (k == 2 ? 0.9749279121818236070181317f : 0.4338837391175581204757683f);
  } else if constexpr (R == 11) {
    switch (k) {
      case 1: return 0.5406408174555975821076360f;
      case 2: return 0.9096319953545183714117154f;
      case 3: return 0.9898214418809327323760920f;
      case 4: return 0.7557495743542582837740358f;
      default: return 0.2817325568414296977114179f;
    }
  } else {
    static_assert(R == 13, "radix");
    switch (k) {
      case 1: return 0.4647231720437685456560153f;
      case 2: return 0.8229838658936563945796174f;
      case 3: return 0.9927088740980539928007516f;
      case 4: return 0.9350162426854148234397846f;
      case 5: return 0.6631226582407952023767855f;
      default: return 0.2393156642875577671487537f;
    }
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

constexpr int inv_mod(int a, int m) {
  for (int i = 1; i < m; ++i)
    if ((a * i) % m == 1) return i;
  return 1;
}

template <int R, int S>
__device__ __forceinline__ void dft_small(float2* x);

// R = A*B with A, B coprime, by the prime-factor index maps (no twiddles):
// input n = (B n1 + A n2) mod R, output k = (B (B^-1 mod A) k1 + A (A^-1 mod B) k2)
// mod R, so that W_R^{nk} = W_A^{n1 k1} W_B^{n2 k2} (Good's mapping; the
// two-factor split of [Mota] section 2.3.1 without its twiddle factors).
template <int A, int B, int S>
__device__ __forceinline__ void dft_pfa(float2* x) {
  constexpr int R = A * B;
  constexpr int BI = inv_mod(B % A, A), AI = inv_mod(A % B, B);
  float2 y[A][B];
  static_for<0, B>([&](auto n2c) {
    constexpr int n2 = decltype(n2c)::value;
    float2 t[A];
    static_for<0, A>([&](auto n1c) {
      constexpr int n1 = decltype(n1c)::value;
      t[n1] = x[(B * n1 + A * n2) % R];
    });
    dft_small<A, S>(t);
#pragma unroll
    for (int k1 = 0; k1 < A; ++k1) y[k1][n2] = t[k1];
  });
  static_for<0, A>([&](auto k1c) {
    constexpr int k1 = decltype(k1c)::value;
    float2 t[B];
#pragma unroll
    for (int n2 = 0; n2 < B; ++n2) t[n2] = y[k1][n2];
    dft_small<B, S>(t);
    static_for<0, B>([&](auto k2c) {
      constexpr int k2 = decltype(k2c)::value;
      x[(B * BI * k1 + A * AI * k2) % R] = t[k2];
    });
  });
}

template <int R, int S>
__device__ __forceinline__ void dft_small(float2* x) {
  if constexpr (R == 2 || R == 4 || R == 8 || R == 16) {
    dft<R, S>(x);
  } else if constexpr (R == 3 || R == 5 || R == 7 || R == 11 || R == 13) {
    dft_prime<R, S>(x);
  } else if constexpr (R == 6) {
    dft_pfa<2, 3, S>(x);
  } else if constexpr (R == 10) {
    dft_pfa<2, 5, S>(x);
  } else if constexpr (R == 12) {
    dft_pfa<4, 3, S>(x);
  } else if constexpr (R == 14) {
    dft_pfa<2, 7, S>(x);
  } else {
    static_assert(R == 15, "radix");
    dft_pfa<3, 5, S>(x);
  }
}

// LDS index of element i of a line: with PAD one pad element after every 32
// elements.  The stage reads are runs of consecutive elements starting at
// offsets r*m that are rarely multiples of 32, which a pad splits; the
// first-stage writes are R elements apart, which a pad spreads over the banks
// when R = 16.  The plan chooses; the choice is compiled in (as a runtime
// shift it cost 4-9 %: no immediate LDS offsets).
template <bool PAD>
__host__ __device__ __forceinline__ uint32_t mixed_pad(uint32_t i) { return PAD ? i + (i >> 5) : i; }
// LDS elements of one Rader line of N values: the padded line, x_0 and A_0
__host__ __device__ __forceinline__ uint32_t rader_line(uint32_t N, bool pad) {
  return (pad ? mixed_pad<true>(N) : mixed_pad<false>(N)) + 2;
}
}  // namespace

// One stage of radix R (compile-time, so the butterfly loops are straight
// code): KB butterflies per thread, b = t + tpl*i.  The first stage gathers
// its inputs from HBM (times pre, or sign-flipped at odd indices when flip
// is set), the others from the line in LDS; the last stage stores to HBM,
// the others back to LDS.  IO bit 1: the first stage reads the line in LDS
// too; IO bit 2: the last stage writes the line in LDS in natural order
// (transforms whose input and output stay on chip).  TWL: the twiddles come
// from twl, the table's copy in LDS, instead of a.tw.
template <int S, int KB, int R, bool PAD, int IO = 0, bool TWL = false>
__device__ __forceinline__ void mixed_stage(const MixedArgs& a, int s, bool last, uint32_t t, uint32_t tpl,
                                            bool valid, const float2* src, float2* dst, float2* L,
                                            const float2* twl) {
  const uint32_t ns = (uint32_t)a.ns[s], m = (uint32_t)a.m[s];
  float2 x[KB][R];
  // gather the inputs of this thread's butterflies: b + r*m
  if (s == 0 && !(IO & 1)) {
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const uint32_t b = t + tpl * i;
      if (valid && b < m) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float2 v = gload_nt(src, b + r * m);
          if (a.pre) v = cmul(v, gload(a.pre, b + r * m));
          if (a.flip && ((b + r * m) & 1)) v = negate_bits(v);
          x[i][r] = v;
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const uint32_t b = t + tpl * i;
      if (b < m) {
#pragma unroll
        for (int r = 0; r < R; ++r) x[i][r] = L[mixed_pad<PAD>(b + r * m)];
      }
    }
    lds_barrier();  // every read of this stage precedes its writes
  }
  // twiddles and the R-point DFTs
#pragma unroll
  for (int i = 0; i < KB; ++i) {
    const uint32_t b = t + tpl * i;
    if (b < m) {
      if (s > 0) {
        const uint32_t j = b - __umulhi(b, a.ns_magic[s]) * ns;
        const float2* tw = (TWL ? twl : a.tw) + a.twoff[s] + j;
#pragma unroll
        for (int r = 1; r < R; ++r) x[i][r] = apply_tw<S>(x[i][r], tw[(r - 1) * ns]);
      }
      dft_small<R, S>(x[i]);
    }
  }
  // scatter the outputs: (b - j) R + j + q ns
  if (!last) {
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const uint32_t b = t + tpl * i;
      if (b < m) {
        const uint32_t j = ns == 1 ? 0u : b - __umulhi(b, a.ns_magic[s]) * ns;
        const uint32_t base = (b - j) * (uint32_t)R + j;
#pragma unroll
        for (int r = 0; r < R; ++r) L[mixed_pad<PAD>(base + r * ns)] = x[i][r];
      }
    }
    lds_barrier();
  } else if constexpr ((IO & 2) != 0) {
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const uint32_t b = t + tpl * i;
      if (b < m) {
#pragma unroll
        for (int r = 0; r < R; ++r) L[mixed_pad<PAD>(b + r * ns)] = x[i][r];
      }
    }
    lds_barrier();
  } else if (valid) {
    // last stage: ns = m and j = b, so output q of butterfly b is b + q m
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const uint32_t b = t + tpl * i;
      if (b < m) {
#pragma unroll
        for (int r = 0; r < R; ++r) gstore_nt(dst, b + r * ns, x[i][r]);
      }
    }
  }
}

// Every stage of the schedule, each compiled for its radix (a switch on the
// schedule's radix selects it; radices 2..8, and with RMAX = 16 also 10..16).
// TWL: the stage twiddles are read from a copy of the table in LDS (twl, the
// same layout as a.tw) instead of HBM/L2; kernels that run several lines per
// workgroup copy the table once for all of them.  The twiddle gathers, not
// the data, kept the texture units busy: with them replaced by register
// values (a timing copy, wrong results) the 1000-point row kernel ran 218 ->
// 180 us per 512 MiB and the four-step of 10^6 717 -> 615 us.
template <int S, int KB, int RMAX, bool PAD, int IO, bool TWL = false>
__device__ __forceinline__ void mixed_stages(const MixedArgs& a, uint32_t t, uint32_t tpl, bool valid,
                                             const float2* src, float2* dst, float2* L,
                                             const float2* twl = nullptr) {
  for (int s = 0; s < a.nstages; ++s) {
    const bool last = s + 1 == a.nstages;
#define FFTAMD_STAGE(R) mixed_stage<S, KB, R, PAD, IO, TWL>(a, s, last, t, tpl, valid, src, dst, L, twl)
    switch (a.radix[s]) {
      case 2: FFTAMD_STAGE(2); break;
      case 3: FFTAMD_STAGE(3); break;
      case 4: FFTAMD_STAGE(4); break;
      case 5: FFTAMD_STAGE(5); break;
      case 6: FFTAMD_STAGE(6); break;
      case 7: FFTAMD_STAGE(7); break;
      case 8: FFTAMD_STAGE(8); break;
      default:
        if constexpr (RMAX > 8) {
          switch (a.radix[s]) {
            case 10: FFTAMD_STAGE(10); break;
            case 11: FFTAMD_STAGE(11); break;
            case 12: FFTAMD_STAGE(12); break;
            case 13: FFTAMD_STAGE(13); break;
            case 14: FFTAMD_STAGE(14); break;
            case 15: FFTAMD_STAGE(15); break;
            default: FFTAMD_STAGE(16); break;
          }
        }
        break;
    }
#undef FFTAMD_STAGE
  }
}

// KB butterflies of at most RMAX values per thread and stage (2 x 8 or
// 1 x 16), up to 1024 threads (so at most 128 VGPRs).  STG: HBM accessed
// through the LDS lines in the block's order (lines of few threads).  TWL
// (with STG): the stage twiddles copied to LDS after the lines, gathered
// before the rows' loads and written to LDS after them so that the two
// latencies overlap.
template <int S, int KB, int RMAX, bool PAD, bool STG, bool TWL = false>
__global__ __launch_bounds__(1024) void k_mixed(MixedArgs a) {
  extern __shared__ float4 smem4[];
  float2* smem = reinterpret_cast<float2*>(smem4);
  // stage twiddles: (R_s - 1) ns_s entries for every stage s >= 1, n - R_0 in all
  const uint32_t ntw = TWL ? (uint32_t)(a.n - a.radix[0]) : 0u;
  lds_poison_dynamic(smem, ((uint32_t)a.lines * (mixed_pad<PAD>((uint32_t)a.n) + 1) + ntw) * sizeof(float2));
  const uint32_t tpl = (uint32_t)a.tpl;
  const int tid = threadIdx.x;
  const int line = tid / (int)tpl;
  const uint32_t t = (uint32_t)(tid - line * (int)tpl);
  const int64_t row = (int64_t)blockIdx.x * a.lines + line;
  const bool valid = row < a.rows;
  const uint32_t n = (uint32_t)a.n;
  const uint32_t lp = mixed_pad<PAD>(n) + 1;
  float2* L = smem + (size_t)line * lp;
  if constexpr (STG) {
    // short lines: the workgroup's rows (one contiguous block) are read and
    // written in order through the lines in LDS; the shift factors apply as
    // the values enter LDS, and the stages run with IO = 3 (line in, line out)
    const int64_t row0 = (int64_t)blockIdx.x * a.lines;
    const int64_t left = a.rows - row0;
    const uint32_t nblk = (uint32_t)(left < a.lines ? left : a.lines) * n;
    const uint32_t NT = tpl * (uint32_t)a.lines;
    const uint32_t magic = 0xffffffffu / n + 1u;  // e / n for e < 2^32 / n
    const float2* src = a.in + row0 * n;
    float2* twl = smem + (uint32_t)a.lines * lp;
    float2 tw0 = make_float2(0.f, 0.f), tw1 = tw0;
    if constexpr (TWL) {
      if ((uint32_t)tid < ntw) tw0 = gload(a.tw, (uint32_t)tid);
      if ((uint32_t)tid + NT < ntw) tw1 = gload(a.tw, (uint32_t)tid + NT);
    }
    constexpr int U = 8;
    for (uint32_t e0 = (uint32_t)tid; e0 < nblk; e0 += U * NT) {
      float2 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k)
        if (e0 + k * NT < nblk) v[k] = gload_nt(src, e0 + k * NT);
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const uint32_t e = e0 + k * NT;
        if (e < nblk) {
          const uint32_t q = __umulhi(e, magic), j = e - q * n;
          float2 x = v[k];
          if (a.pre) x = cmul(x, gload(a.pre, j));
          if (a.flip && (j & 1)) x = negate_bits(x);
          smem[q * lp + mixed_pad<PAD>(j)] = x;
        }
      }
    }
    if constexpr (TWL) {
      if ((uint32_t)tid < ntw) twl[tid] = tw0;
      if ((uint32_t)tid + NT < ntw) twl[tid + NT] = tw1;
      for (uint32_t e = (uint32_t)tid + 2 * NT; e < ntw; e += NT) twl[e] = gload(a.tw, e);
    }
    lds_barrier();
    mixed_stages<S, KB, RMAX, PAD, 3, TWL>(a, t, tpl, valid, nullptr, nullptr, L, twl);
    float2* dst = a.out + row0 * n;
    for (uint32_t e = (uint32_t)tid; e < nblk; e += NT) {
      const uint32_t q = __umulhi(e, magic), j = e - q * n;
      gstore_nt(dst, e, smem[q * lp + mixed_pad<PAD>(j)]);
    }
  } else {
    mixed_stages<S, KB, RMAX, PAD, 0>(a, t, tpl, valid, a.in + row * n, a.out + row * n, L);
  }
}

// Rader's transform of a prime length p (see launch.hpp), one line of
// N = p - 1 values in LDS per row: load the row coalesced and place x_j
// (j >= 1) at position (-ind j) mod N, the forward N-point transform, the
// product with conv (A_0 = sum of x_j, j >= 1, kept aside), the inverse
// N-point transform, then X_0 = x_0 + A_0 and X_j = x_0 + c_(ind j), stored
// coalesced.  The pre factors (the shift of odd lengths) apply on load.
// TWL: the stage twiddles of both transforms from a copy in LDS after the
// lines (gathered before the rows' loads, written to LDS after them).
template <int KB, int RMAX, bool PAD, bool STG, bool TWL = false>
__global__ __launch_bounds__(1024) void k_rader(MixedArgs a, RaderArgs rd) {
  extern __shared__ float4 smem4[];
  float2* smem = reinterpret_cast<float2*>(smem4);
  const uint32_t ntw = TWL ? (uint32_t)(a.n - a.radix[0]) : 0u;
  lds_poison_dynamic(smem, ((uint32_t)a.lines * rader_line((uint32_t)a.n, PAD) + ntw) * sizeof(float2));
  float2* twl = smem + (size_t)a.lines * rader_line((uint32_t)a.n, PAD);
  float2 tw0 = make_float2(0.f, 0.f), tw1 = tw0;
  if constexpr (TWL) {
    if (threadIdx.x < ntw) tw0 = gload(a.tw, threadIdx.x);
    if (threadIdx.x + blockDim.x < ntw) tw1 = gload(a.tw, threadIdx.x + blockDim.x);
  }
  const uint32_t tpl = (uint32_t)a.tpl;
  const int tid = threadIdx.x;
  const int line = tid / (int)tpl;
  const uint32_t t = (uint32_t)(tid - line * (int)tpl);
  const int64_t row = (int64_t)blockIdx.x * a.lines + line;
  const bool valid = row < a.rows;
  const uint32_t N = (uint32_t)a.n, p = (uint32_t)rd.p;
  const uint32_t lp = rader_line(N, PAD);
  float2* L = smem + (size_t)line * lp;
  float2* x0s = L + (lp - 2);  // x_0, then A_0
  // STG (lines of few threads): the workgroup's rows, one contiguous block,
  // read and written in order; element e is x_j of line e / p
  const int64_t row0 = (int64_t)blockIdx.x * a.lines;
  const int64_t left = a.rows - row0;
  const uint32_t nblk = (uint32_t)(left < a.lines ? left : a.lines) * p;
  const uint32_t NT = tpl * (uint32_t)a.lines;
  const uint32_t magic = 0xffffffffu / p + 1u;  // e / p for e < 2^32 / p
  if constexpr (STG) {
    const float2* src = a.in + row0 * p;
    constexpr int U = 8;
    for (uint32_t e0 = (uint32_t)tid; e0 < nblk; e0 += U * NT) {
      float2 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k)
        if (e0 + k * NT < nblk) v[k] = gload_nt(src, e0 + k * NT);
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const uint32_t e = e0 + k * NT;
        if (e < nblk) {
          const uint32_t q = __umulhi(e, magic), j = e - q * p;
          float2 x = v[k];
          if (a.pre) x = cmul(x, gload(a.pre, j));
          float2* Lq = smem + (size_t)q * lp;
          Lq[j == 0 ? lp - 2 : mixed_pad<PAD>((uint32_t)rd.perm[j].x)] = x;
        }
      }
    }
  } else if (valid) {
    const float2* src = a.in + row * (int64_t)p;
    for (uint32_t j = t; j < p; j += tpl) {
      float2 v = gload_nt(src, j);
      if (a.pre) v = cmul(v, gload(a.pre, j));
      if (j == 0) {
        x0s[0] = v;
      } else {
        L[mixed_pad<PAD>((uint32_t)rd.perm[j].x)] = v;
      }
    }
  }
  if constexpr (TWL) {
    if (threadIdx.x < ntw) twl[threadIdx.x] = tw0;
    if (threadIdx.x + blockDim.x < ntw) twl[threadIdx.x + blockDim.x] = tw1;
    for (uint32_t e = threadIdx.x + 2 * blockDim.x; e < ntw; e += blockDim.x) twl[e] = gload(a.tw, e);
  }
  lds_barrier();
  mixed_stages<-1, KB, RMAX, PAD, 3, TWL>(a, t, tpl, valid, nullptr, nullptr, L, twl);
  for (uint32_t k = t; k < N; k += tpl) {
    const float2 A = L[mixed_pad<PAD>(k)];
    if (k == 0) x0s[1] = A;
    L[mixed_pad<PAD>(k)] = cmul(A, gload(rd.conv, k));
  }
  lds_barrier();
  mixed_stages<1, KB, RMAX, PAD, 3, TWL>(a, t, tpl, valid, nullptr, nullptr, L, twl);
  if constexpr (STG) {
    float2* dst = a.out + row0 * p;
    for (uint32_t e = (uint32_t)tid; e < nblk; e += NT) {
      const uint32_t q = __umulhi(e, magic), j = e - q * p;
      const float2* Lq = smem + (size_t)q * lp;
      const float2 x0 = Lq[lp - 2];
      const float2 c = Lq[j == 0 ? lp - 1 : mixed_pad<PAD>((uint32_t)rd.perm[j].y)];
      gstore_nt(dst, e, make_float2(x0.x + c.x, x0.y + c.y));
    }
  } else if (valid) {
    float2* dst = a.out + row * (int64_t)p;
    const float2 x0 = x0s[0];
    for (uint32_t j = t; j < p; j += tpl) {
      const float2 c = j == 0 ? x0s[1] : L[mixed_pad<PAD>((uint32_t)rd.perm[j].y)];
      gstore_nt(dst, j, make_float2(x0.x + c.x, x0.y + c.y));
    }
  }
}

// Bluestein's chirp transform on a convolution length m with a mixed-radix
// schedule: the row times pre, zero beyond n, as a line of m values in LDS;
// the forward m-point stages; the product with bhat; the inverse stages; the
// outputs j < n times post.  STG: the rows read and written as one block.
// TWL: the stage twiddles of both transforms from a copy in LDS, as in k_rader.
template <bool PAD, bool STG, bool TWL = false>
__global__ __launch_bounds__(1024) void k_bluestein_mixed(MixedArgs a, ChirpMixedArgs c) {
  extern __shared__ float4 smem4[];
  float2* smem = reinterpret_cast<float2*>(smem4);
  const uint32_t ntw = TWL ? (uint32_t)(a.n - a.radix[0]) : 0u;
  lds_poison_dynamic(smem, ((uint32_t)a.lines * (mixed_pad<PAD>((uint32_t)a.n) + 1) + ntw) * sizeof(float2));
  float2* twl = smem + (size_t)a.lines * (mixed_pad<PAD>((uint32_t)a.n) + 1);
  float2 tw0 = make_float2(0.f, 0.f), tw1 = tw0;
  if constexpr (TWL) {
    if (threadIdx.x < ntw) tw0 = gload(a.tw, threadIdx.x);
    if (threadIdx.x + blockDim.x < ntw) tw1 = gload(a.tw, threadIdx.x + blockDim.x);
  }
  const uint32_t tpl = (uint32_t)a.tpl;
  const int tid = threadIdx.x;
  const int line = tid / (int)tpl;
  const uint32_t t = (uint32_t)(tid - line * (int)tpl);
  const int64_t row = (int64_t)blockIdx.x * a.lines + line;
  const bool valid = row < a.rows;
  const uint32_t m = (uint32_t)a.n, n = (uint32_t)c.n;
  const uint32_t lp = mixed_pad<PAD>(m) + 1;
  float2* L = smem + (size_t)line * lp;
  // STG (lines of few threads): the workgroup's rows, one contiguous block of
  // n-value rows, read and written in order; element e is x_j of line e / n
  const int64_t row0 = (int64_t)blockIdx.x * a.lines;
  const int64_t left = a.rows - row0;
  const uint32_t nblk = (uint32_t)(left < a.lines ? left : a.lines) * n;
  const uint32_t NT = tpl * (uint32_t)a.lines;
  const uint32_t magic = 0xffffffffu / n + 1u;  // e / n for e < 2^32 / n
  if constexpr (STG) {
    const float2* src = a.in + row0 * n;
    constexpr int U = 8;
    for (uint32_t e0 = (uint32_t)tid; e0 < nblk; e0 += U * NT) {
      float2 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k)
        if (e0 + k * NT < nblk) v[k] = gload_nt(src, e0 + k * NT);
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const uint32_t e = e0 + k * NT;
        if (e < nblk) {
          const uint32_t q = __umulhi(e, magic), j = e - q * n;
          smem[q * lp + mixed_pad<PAD>(j)] = cmul(v[k], gload(a.pre, j));
        }
      }
    }
    for (uint32_t j = n + t; j < m; j += tpl) L[mixed_pad<PAD>(j)] = make_float2(0.f, 0.f);
  } else {
    const float2* src = a.in + row * (int64_t)n;
    for (uint32_t j = t; j < m; j += tpl) {
      float2 v = make_float2(0.f, 0.f);
      if (valid && j < n) v = cmul(gload_nt(src, j), gload(a.pre, j));
      L[mixed_pad<PAD>(j)] = v;
    }
  }
  if constexpr (TWL) {
    if (threadIdx.x < ntw) twl[threadIdx.x] = tw0;
    if (threadIdx.x + blockDim.x < ntw) twl[threadIdx.x + blockDim.x] = tw1;
    for (uint32_t e = threadIdx.x + 2 * blockDim.x; e < ntw; e += blockDim.x) twl[e] = gload(a.tw, e);
  }
  lds_barrier();
  mixed_stages<-1, 1, 16, PAD, 3, TWL>(a, t, tpl, valid, nullptr, nullptr, L, twl);
  for (uint32_t k = t; k < m; k += tpl) L[mixed_pad<PAD>(k)] = cmul(L[mixed_pad<PAD>(k)], gload(c.bhat, k));
  lds_barrier();
  mixed_stages<1, 1, 16, PAD, 3, TWL>(a, t, tpl, valid, nullptr, nullptr, L, twl);
  if constexpr (STG) {
    float2* dst = a.out + row0 * n;
    for (uint32_t e = (uint32_t)tid; e < nblk; e += NT) {
      const uint32_t q = __umulhi(e, magic), j = e - q * n;
      gstore_nt(dst, e, cmul(smem[q * lp + mixed_pad<PAD>(j)], gload(c.post, j)));
    }
  } else if (valid) {
    float2* dst = a.out + row * (int64_t)n;
    for (uint32_t j = t; j < n; j += tpl) gstore_nt(dst, j, cmul(L[mixed_pad<PAD>(j)], gload(c.post, j)));
  }
}

// Column transforms of a mixed-radix length over [images][n][nx] (see
// launch.hpp, launch_mixed_cols): CT adjacent columns of the flattened
// images x nx column index per workgroup.  Load: consecutive threads on
// consecutive columns, so each row of the tile is one run of CT values,
// into line `column` of LDS at the row's position (the shift applied on
// load); then the stages with the line in LDS (IO = 3: the first stage
// reads it, the last writes it back in natural order), G lines at a time
// with tpl threads each (threads beyond the group's lines take no butterfly
// but join every barrier); then the columns are stored back.
// 8 loads (and 8 twiddle pairs) in flight per thread: 60-64 VGPRs, 8 waves
// per SIMD; with 16, 108-123 VGPRs and 4 waves cost per 512 MiB: 2D 360 x
// 360 494 against 652 us, 125 x 160 460 against 595, 12 x 4096 369 against
// 473; the four-step of 20000 794 against 965, 6561 997 against 1279
constexpr int kColBatch = 8;
// TROWS: the tile is CT consecutive rows (contiguous, read in order) whose
// transforms are stored transposed (launch_mixed_rows_t).
// LONG (lines of 512 points and more, 8 per workgroup): at most 64 VGPRs (a
// few spilled dwords in the padded forms) and the loads issued at raised
// wave priority.  Per 512 MiB: the four-step of 10^6 (1000-point tiles in
// both passes) 801 -> 718 us, of 3 * 2^20 (1024-point columns) 925 -> 846,
// 2D 1000 x 1000 546 -> 539; for shorter lines (128-400 points: 24576,
// 49152, 160000, 2D 360 x 360) the same settings cost up to 3 %.
// TWL: the stage twiddles in LDS after the CT lines (tile_shape decides).
// FSL (with TWL, column tiles of the four-step): thi and tlo in LDS after
// them, the entries the tile's exponents x k < n nx can reach.
template <int S, int KB, int RMAX, bool PAD, bool TROWS, bool LONG, bool TWL, bool FSL = false>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(LONG ? 8 : 1))) void k_mixed_cols(MixedArgs a, MixedColsArgs c) {
  extern __shared__ float4 smem4[];
  float2* smem = reinterpret_cast<float2*>(smem4);
  const uint32_t n = (uint32_t)a.n, tpl = (uint32_t)a.tpl, nt = blockDim.x, tid = threadIdx.x;
  const uint32_t CT = (uint32_t)a.lines;  // columns per workgroup (set by the launcher)
  const uint32_t pitch = mixed_pad<PAD>(n) + 1;
  // stage twiddles: (R_s - 1) ns_s entries for every stage s >= 1, n - R_0 in all
  const uint32_t ntw = TWL ? (uint32_t)(a.n - a.radix[0]) : 0u;
  const uint32_t nhi = FSL ? (((uint32_t)(a.n - 1) * (uint32_t)(c.nx - 1)) >> c.bits) + 1u : 0u;
  const uint32_t nlo = FSL ? 1u << c.bits : 0u;
  lds_poison_dynamic(smem, (CT * pitch + ntw + nhi + nlo) * (uint32_t)sizeof(float2));
  float2* twl = smem + CT * pitch;
  float2* hil = twl + ntw;
  float2* lol = hil + nhi;
  float2 th0 = make_float2(0.f, 0.f), tl0 = th0;
  if constexpr (FSL) {
    if (tid < nhi) th0 = gload(c.thi, tid);
    if (tid < nlo) tl0 = gload(c.tlo, tid);
  }
  // the table's first 2 * nt entries are gathered before the tile's loads
  // and written to LDS after them, so that its latency overlaps theirs
  float2 tw0 = make_float2(0.f, 0.f), tw1 = tw0;
  if constexpr (TWL) {
    if (tid < ntw) tw0 = gload(a.tw, tid);
    if (tid + nt < ntw) tw1 = gload(a.tw, tid + nt);
  }
  // thread tid takes column tid % CT of the tile and rows tid / CT + RS*i
  // (nt is a multiple of 64, so of CT): one division per thread, and
  // kColBatch loads in flight before their LDS writes
  const uint32_t col = tid % CT, RS = nt / CT;
  const int64_t g = (int64_t)blockIdx.x * CT + col;
  const bool has_col = g < c.images * c.nx;
  const int64_t img = g / c.nx;
  float2* L0 = smem + col * pitch;
  if constexpr (TROWS) {
    // rows g0 .. g0 + CT - 1, one contiguous block: element e is entry e % n
    // of line e / n
    const int64_t g0 = (int64_t)blockIdx.x * CT, left = c.images * c.nx - g0;
    const uint32_t nblk = (uint32_t)(left < (int64_t)CT ? left : (int64_t)CT) * n;
    const uint32_t magic = 0xffffffffu / n + 1u;  // e / n for e < 2^32 / n
    const float2* blk = a.in + g0 * n;
    if constexpr (LONG) __builtin_amdgcn_s_setprio(3);
    for (uint32_t e0 = tid; e0 < nblk; e0 += kColBatch * nt) {
      float2 v[kColBatch];
#pragma unroll
      for (int i = 0; i < kColBatch; ++i)
        if (e0 + i * nt < nblk) v[i] = gload_nt(blk, e0 + i * nt);
#pragma unroll
      for (int i = 0; i < kColBatch; ++i) {
        const uint32_t e = e0 + i * nt;
        if (e < nblk) {
          const uint32_t q = __umulhi(e, magic);
          smem[q * pitch + mixed_pad<PAD>(e - q * n)] = v[i];
        }
      }
    }
    if constexpr (LONG) __builtin_amdgcn_s_setprio(0);
  } else {
  const float2* src = a.in + img * (int64_t)n * c.nx + (g - img * c.nx);
  if constexpr (LONG) __builtin_amdgcn_s_setprio(3);
  for (uint32_t r0 = tid / CT; r0 < n; r0 += kColBatch * RS) {
    float2 v[kColBatch];
#pragma unroll
    for (int i = 0; i < kColBatch; ++i) {
      const uint32_t r = r0 + RS * i;
      v[i] = make_float2(0.f, 0.f);
      if (has_col && r < n) {
        v[i] = gload(src, r * (uint32_t)c.nx);
        if (a.pre) v[i] = cmul(v[i], gload(a.pre, r));
        if (a.flip && (r & 1)) v[i] = negate_bits(v[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < kColBatch; ++i) {
      const uint32_t r = r0 + RS * i;
      if (r < n) L0[mixed_pad<PAD>(r)] = v[i];
    }
  }
  if constexpr (LONG) __builtin_amdgcn_s_setprio(0);
  }
  if constexpr (TWL) {
    if (tid < ntw) twl[tid] = tw0;
    if (tid + nt < ntw) twl[tid + nt] = tw1;
    for (uint32_t e = tid + 2 * nt; e < ntw; e += nt) twl[e] = gload(a.tw, e);
  }
  if constexpr (FSL) {
    if (tid < nhi) hil[tid] = th0;
    if (tid < nlo) lol[tid] = tl0;
    for (uint32_t e = tid + nt; e < nhi; e += nt) hil[e] = gload(c.thi, e);
    for (uint32_t e = tid + nt; e < nlo; e += nt) lol[e] = gload(c.tlo, e);
  }
  lds_barrier();
  const uint32_t G = nt / tpl;  // lines per group
  for (uint32_t l0 = 0; l0 < CT; l0 += G) {
    const uint32_t line = l0 + tid / tpl;
    const bool active = tid < G * tpl && line < CT;
    // an inactive thread's butterfly index is past every stage's count
    mixed_stages<S, KB, RMAX, PAD, 3, TWL>(a, active ? tid % tpl : 0x40000000u, tpl, active, nullptr, nullptr,
                                           smem + (active ? line : 0u) * pitch, twl);
  }
  if constexpr (TROWS) {
    // line col is row k2 = g - img * nx of image img; entry k1 goes to
    // (k1 * nx + k2 + rot) mod (n * nx): the CT lines of one k1 are a run
    // Streaming stores where a run is whole 128 B lines; ordinary ones where
    // runs straddle lines (nx not a multiple of 16), so that the L2 merges
    // the halves two workgroups write (n = 20000, runs 1000 B apart: 854 ->
    // 696 us per 512 MiB; aligned runs 1-5 % slower that way)
    if (has_col) {
      const uint32_t k2 = (uint32_t)(g - img * c.nx), nx = (uint32_t)c.nx, len = n * nx;
      const bool whole = CT == 16 && nx % 16 == 0;
      float2* dst = a.out + img * (int64_t)len;
      for (uint32_t k1 = tid / CT; k1 < n; k1 += RS) {
        uint32_t e = k1 * nx + k2 + (uint32_t)c.rot;
        if (e >= len) e -= len;
        if (whole)
          gstore_nt(dst, e, L0[mixed_pad<PAD>(k1)]);
        else
          gstore(dst, e, L0[mixed_pad<PAD>(k1)]);
      }
    }
  } else if (has_col && c.thi) {
    // the four-step's W^{x k}: kColBatch pairs of table loads in flight
    // before their stores
    float2* dst = a.out + img * (int64_t)n * c.nx + (g - img * c.nx);
    const uint32_t x = (uint32_t)(g - img * c.nx), mask = (1u << c.bits) - 1u;
    for (uint32_t r0 = tid / CT; r0 < n; r0 += kColBatch * RS) {
      float2 wh[kColBatch], wl[kColBatch];
#pragma unroll
      for (int i = 0; i < kColBatch; ++i) {
        const uint32_t r = r0 + RS * i, e = x * r;
        if (r < n) {
          if constexpr (FSL) {
            wh[i] = hil[e >> c.bits];
            wl[i] = lol[e & mask];
          } else {
            wh[i] = gload(c.thi, e >> c.bits);
            wl[i] = gload(c.tlo, e & mask);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kColBatch; ++i) {
        const uint32_t r = r0 + RS * i;
        if (r < n) gstore(dst, r * (uint32_t)c.nx, apply_tw<S>(L0[mixed_pad<PAD>(r)], cmul(wh[i], wl[i])));
      }
    }
  } else if (has_col) {
    float2* dst = a.out + img * (int64_t)n * c.nx + (g - img * c.nx);
    for (uint32_t r = tid / CT; r < n; r += RS) gstore(dst, r * (uint32_t)c.nx, L0[mixed_pad<PAD>(r)]);
  }
}

namespace {
// the checks every launch of a schedule needs (host side, before any HIP call)
bool mixed_schedule_ok(const MixedArgs& a, int* rmax_out) {
  if (a.n < 2 || a.n > kMaxMixedLength || a.nstages < 1 || a.nstages > kMixedMaxStages || a.tpl < 1 ||
      a.lines < 1 || a.tpl * a.lines > 1024 || a.rows < 1 || (a.kb != 1 && a.kb != 2) || (a.pad != 0 && a.pad != 1))
    return false;
  int rmax = 0;
  for (int s = 0; s < a.nstages; ++s) {
    const int R = a.radix[s];
    if (R < 2 || R > 16 || R == 9) return false;
    if ((int64_t)a.tpl * a.kb < a.m[s]) return false;  // every butterfly has a thread
    rmax = R > rmax ? R : rmax;
  }
  *rmax_out = rmax;
  return true;
}
}  // namespace

namespace {
template <bool TWL>
hipError_t launch_mixed_stg(int sign, int rmax, const MixedArgs& a, dim3 grid, dim3 block, size_t lds, hipStream_t st) {
  if (rmax > 8) {
    if (a.pad) {
      if (sign < 0)
        FFTAMD_LAUNCH((k_mixed<-1, 1, 16, true, true, TWL>), grid, block, lds, st, a);
      else
        FFTAMD_LAUNCH((k_mixed<1, 1, 16, true, true, TWL>), grid, block, lds, st, a);
    } else if (sign < 0) {
      FFTAMD_LAUNCH((k_mixed<-1, 1, 16, false, true, TWL>), grid, block, lds, st, a);
    } else {
      FFTAMD_LAUNCH((k_mixed<1, 1, 16, false, true, TWL>), grid, block, lds, st, a);
    }
  } else if (a.pad) {
    return hipErrorInvalidValue;
  } else if (sign < 0) {
    FFTAMD_LAUNCH((k_mixed<-1, 2, 8, false, true, TWL>), grid, block, lds, st, a);
  } else {
    FFTAMD_LAUNCH((k_mixed<1, 2, 8, false, true, TWL>), grid, block, lds, st, a);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_mixed(int sign, const MixedArgs& a, hipStream_t st) {
  int rmax = 0;
  if (!mixed_schedule_ok(a, &rmax)) return hipErrorInvalidValue;
  uint32_t grid;
  hipError_t e = grid_of(a.rows, a.lines, &grid);
  if (e != hipSuccess) return e;
  const size_t lds =
      (size_t)a.lines * ((a.pad ? mixed_pad<true>((uint32_t)a.n) : mixed_pad<false>((uint32_t)a.n)) + 1) * sizeof(float2);
  if (lds > (size_t)kLdsBudgetBytes) return hipErrorInvalidValue;
  const dim3 block((uint32_t)(a.tpl * a.lines));
  // Lines of fewer than 128 threads read and write HBM through LDS (STG): a
  // butterfly's direct loads are runs of m[0] elements, as short as one.
  // Per 512 MiB: n = 3 261 -> 166 us, 6 1124 -> 171, 12 2799 -> 174, 15 3566
  // -> 228, 24 383 -> 183, 48 267 -> 173, 100 300 -> 187, 360 233 -> 207,
  // 1000 232 -> 225.  So do one-butterfly lines of 800 threads and more (one
  // line per workgroup): 4000 416 -> 382, 4500 459 -> 359, 5000 380 -> 293,
  // 6000 361 -> 281, 7000 339 -> 272, 8000 329 -> 263.  Lines of 128 to 768
  // threads were 3-15 % slower staged (1296, 2000, 2187, 3000, 3125, 3500,
  // 4200, 4320, 5120, 6144), and so were two-butterfly lines (7200, 7776).
  if (a.n <= 8192 && (a.tpl < 128 || (a.tpl >= 800 && a.kb == 1))) {
    // the stage twiddles in LDS where a workgroup holds 3 lines or more (per
    // 512 MiB: n = 360 207 -> 183 us, 500 267 -> 232, 100 186 -> 180, 48 173
    // -> 170, 768 and 2000 unchanged); with 2 lines the larger LDS share costs
    // more than it saves (1000: 219 -> 231 us), so those run 4 lines
    const size_t ldst = lds + (size_t)(a.n - a.radix[0]) * sizeof(float2);
    if (a.lines >= 3 && ldst <= (size_t)kLdsBudgetBytes)
      return launch_mixed_stg<true>(sign, rmax, a, dim3(grid), block, ldst, st);
    // two lines per workgroup become four with the table (1000: 220 -> 212
    // us; 2D 1000 x 1000 522 -> 508, 1000 x 600 544 -> 525; 2000 unchanged)
    if (a.lines == 2 && a.tpl * 4 <= 1024) {
      MixedArgs a4 = a;
      a4.lines = 4;
      uint32_t grid4;
      e = grid_of(a4.rows, a4.lines, &grid4);
      if (e != hipSuccess) return e;
      const size_t lds4 = 2 * lds + (size_t)(a.n - a.radix[0]) * sizeof(float2);
      if (lds4 <= (size_t)kLdsBudgetBytes)
        return launch_mixed_stg<true>(sign, rmax, a4, dim3(grid4), dim3((uint32_t)(a4.tpl * 4)), lds4, st);
    }
    return launch_mixed_stg<false>(sign, rmax, a, dim3(grid), block, lds, st);
  }
  if (rmax > 8 && a.kb == 2) {
    // lengths above 8192: two butterflies of up to 16 values per thread
    if (a.pad) return hipErrorInvalidValue;
    if (sign < 0)
      FFTAMD_LAUNCH((k_mixed<-1, 2, 16, false, false>), dim3(grid), block, lds, st, a);
    else
      FFTAMD_LAUNCH((k_mixed<1, 2, 16, false, false>), dim3(grid), block, lds, st, a);
  } else if (rmax > 8) {
    if (a.pad) {
      if (sign < 0)
        FFTAMD_LAUNCH((k_mixed<-1, 1, 16, true, false>), dim3(grid), block, lds, st, a);
      else
        FFTAMD_LAUNCH((k_mixed<1, 1, 16, true, false>), dim3(grid), block, lds, st, a);
    } else if (sign < 0) {
      FFTAMD_LAUNCH((k_mixed<-1, 1, 16, false, false>), dim3(grid), block, lds, st, a);
    } else {
      FFTAMD_LAUNCH((k_mixed<1, 1, 16, false, false>), dim3(grid), block, lds, st, a);
    }
  } else if (a.pad) {
    return hipErrorInvalidValue;  // schedules of radices up to 8 run unpadded
  } else if (sign < 0) {
    FFTAMD_LAUNCH((k_mixed<-1, 2, 8, false, false>), dim3(grid), block, lds, st, a);
  } else {
    FFTAMD_LAUNCH((k_mixed<1, 2, 8, false, false>), dim3(grid), block, lds, st, a);
  }
  return hipGetLastError();
}

// 16 columns (128 B runs) while they take at most 80 KiB of LDS (two
// workgroups per CU) and 16 lines need at most 384 threads, else 8 (64 B
// runs).  One 16-column workgroup per CU was slower (per 512 MiB: 2D 1000 x
// 1000 575 against 544 us, 720 x 720 616 against 564, 640 x 480 590 against
// 516; the four-step of 10^6 883 against 839; 4 * 10^6 992 against 1029 the
// exception), and so were workgroups of more than 384 threads (2D 360 x 360,
// 60 threads per line: 501 against 470 us; 200 x 300 573 against 554; the
// four-step of 6561 876 against 812, of 100000 894 against 799), while
// 8-column tiles of short lines lost (24576, 16 threads per line: 617
// against 448 us; 2D 12 x 4096 519 against 365)
namespace {
// columns per workgroup and whether the stage twiddles (n - R_0 entries)
// fit in LDS beside the tile.  With the table in LDS, per 512 MiB: the
// four-step of 100000 795 -> 663 us, 160000 795 -> 655, 10^6 716 -> 643,
// 2 * 10^6 909 -> 817, 36000 603 -> 542, 49152 499 -> 454, 20000 686 -> 661,
// 6561 804 -> 736; 2D 640 x 480 521 -> 468, 720 x 720 561 -> 518, 360 x 360
// 466 -> 448, 1000 x 1000 538 -> 521; 15625 (125-point tiles both ways) the
// exception, 737 -> 773
int tile_shape(const MixedArgs& a, bool* twl) {
  const size_t pitch = (size_t)(a.pad ? mixed_pad<true>((uint32_t)a.n) : mixed_pad<false>((uint32_t)a.n)) + 1;
  const size_t tw = (size_t)(a.n - a.radix[0]);
  *twl = true;
  if ((16 * pitch + tw) * sizeof(float2) <= 81920 && 16 * a.tpl <= 384) return 16;
  if ((8 * pitch + tw) * sizeof(float2) <= (size_t)kLdsBudgetBytes) return 8;
  *twl = false;
  if (8 * pitch * sizeof(float2) <= (size_t)kLdsBudgetBytes) return 8;
  return 0;
}
}  // namespace

int mixed_cols_tile(const MixedArgs& a) {
  bool twl = false;
  return tile_shape(a, &twl);
}

namespace {
// the compiled tile kernel of one schedule shape
template <bool TROWS, bool LONG, bool TWL, bool FSL = false>
hipError_t launch_tiles_k(int sign, int rmax, bool pad, dim3 grid, dim3 block, size_t lds, hipStream_t st,
                          const MixedArgs& a, const MixedColsArgs& c) {
  if (rmax > 8) {
    if (pad) {
      if (sign < 0)
        FFTAMD_LAUNCH((k_mixed_cols<-1, 1, 16, true, TROWS, LONG, TWL, FSL>), grid, block, lds, st, a, c);
      else
        FFTAMD_LAUNCH((k_mixed_cols<1, 1, 16, true, TROWS, LONG, TWL, FSL>), grid, block, lds, st, a, c);
    } else if (sign < 0) {
      FFTAMD_LAUNCH((k_mixed_cols<-1, 1, 16, false, TROWS, LONG, TWL, FSL>), grid, block, lds, st, a, c);
    } else {
      FFTAMD_LAUNCH((k_mixed_cols<1, 1, 16, false, TROWS, LONG, TWL, FSL>), grid, block, lds, st, a, c);
    }
  } else if (pad) {
    return hipErrorInvalidValue;  // schedules of radices up to 8 run unpadded
  } else if (sign < 0) {
    FFTAMD_LAUNCH((k_mixed_cols<-1, 2, 8, false, TROWS, LONG, TWL, FSL>), grid, block, lds, st, a, c);
  } else {
    FFTAMD_LAUNCH((k_mixed_cols<1, 2, 8, false, TROWS, LONG, TWL, FSL>), grid, block, lds, st, a, c);
  }
  return hipGetLastError();
}

template <bool TROWS>
hipError_t launch_tiles(int sign, const MixedArgs& a0, const MixedColsArgs& c, hipStream_t st) {
  int rmax = 0;
  MixedArgs a = a0;
  a.rows = 1;
  a.lines = 1;
  if (!mixed_schedule_ok(a, &rmax) || c.nx < 1 || c.images < 1 || !a.in || !a.out) return hipErrorInvalidValue;
  if (rmax > 8 && a.kb != 1) return hipErrorInvalidValue;  // no column-tile kernel of this shape
  if (c.thi && (!c.tlo || c.bits < 1 || c.bits > 16 || (int64_t)a.n * c.nx > (int64_t(1) << 32)))
    return hipErrorInvalidValue;  // the twiddle exponents x k must fit 32 bits
  bool twl = false;
  const int ct = tile_shape(a, &twl);
  if (ct == 0) return hipErrorInvalidValue;
  a.lines = ct;
  const int64_t cols = c.images * c.nx;
  // element offsets r * nx within an image: below 2^29 (gload's 32-bit byte offsets)
  if ((int64_t)a.n * c.nx > (int64_t(1) << 29)) return hipErrorInvalidValue;
  const int64_t blocks = (cols + ct - 1) / ct;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // lines per group: as many as 1024 threads hold, at least 256 threads
  int g = 1024 / a.tpl;
  if (g > ct) g = ct;
  int threads = g * a.tpl;
  threads = (threads + 63) / 64 * 64;
  const size_t pitch = (size_t)(a.pad ? mixed_pad<true>((uint32_t)a.n) : mixed_pad<false>((uint32_t)a.n)) + 1;
  const size_t lds = ((size_t)ct * pitch + (twl ? (size_t)(a.n - a.radix[0]) : 0)) * sizeof(float2);
  const dim3 grid((uint32_t)blocks), block((uint32_t)threads);
  if constexpr (!TROWS) {
    if (twl && c.thi) {
      // the four-step's tables in LDS too for 16-column tiles (the copy shared
      // by 16 columns, the workgroups per CU kept).  Per 512 MiB: 24576 443
      // -> 411 us, 49152 456 -> 421, 36000 549 -> 534; with 8-column tiles
      // the results were mixed (20000 663 -> 630, but 15625 774 -> 791,
      // 100000 667 -> 675, 160000 658 -> 669), so those keep them in HBM
      const size_t nhi = ((((size_t)a.n - 1) * ((size_t)c.nx - 1)) >> c.bits) + 1, nlo = size_t(1) << c.bits;
      const size_t ldsf = lds + (nhi + nlo) * sizeof(float2);
      if (ct == 16 && ldsf <= (lds <= 81920 ? 81920 : (size_t)kLdsBudgetBytes)) {
        if (a.n >= 512) return launch_tiles_k<false, true, true, true>(sign, rmax, a.pad != 0, grid, block, ldsf, st, a, c);
        return launch_tiles_k<false, false, true, true>(sign, rmax, a.pad != 0, grid, block, ldsf, st, a, c);
      }
    }
  }
  if (!twl) return launch_tiles_k<TROWS, true, false>(sign, rmax, a.pad != 0, grid, block, lds, st, a, c);
  if (a.n >= 512) return launch_tiles_k<TROWS, true, true>(sign, rmax, a.pad != 0, grid, block, lds, st, a, c);
  return launch_tiles_k<TROWS, false, true>(sign, rmax, a.pad != 0, grid, block, lds, st, a, c);
}
}  // namespace

hipError_t launch_mixed_cols(int sign, const MixedArgs& a, const MixedColsArgs& c, hipStream_t st) {
  return launch_tiles<false>(sign, a, c, st);
}

hipError_t launch_mixed_rows_t(int sign, const MixedArgs& a, const MixedColsArgs& c, hipStream_t st) {
  if (c.thi || c.rot < 0 || c.rot >= (int64_t)a.n * c.nx || a.in == a.out) return hipErrorInvalidValue;
  return launch_tiles<true>(sign, a, c, st);
}

namespace {
// workgroups per CU that LDS and 8 waves per SIMD allow.  The Rader and
// chirp kernels run two transforms per line on one stage table, so the copy
// in LDS pays even with one line per workgroup, but only while it keeps the
// workgroups per CU (per 512 MiB: Rader p = 97 334 -> 294 us, 257 406 ->
// 366, 641 394 -> 330, 1009 494 -> 457, 3001 676 -> 625, 4001 699 -> 630;
// chirp 34 471 -> 435, 2111 972 -> 906; with fewer workgroups 2017 460 ->
// 618, 6007 540 -> 766, 1034 754 -> 943, 1049 655 -> 857)
int wg_per_cu(size_t lds, uint32_t threads) {
  const int by_waves = 32 / (int)((threads + 63) / 64);
  const int by_lds = lds ? (int)((size_t)kLdsBudgetBytes / lds) : by_waves;
  return by_waves < by_lds ? by_waves : by_lds;
}
}  // namespace

hipError_t launch_rader(const MixedArgs& a, const RaderArgs& rd, hipStream_t st) {
  int rmax = 0;
  if (!mixed_schedule_ok(a, &rmax) || rd.p != a.n + 1 || !rd.conv || !rd.perm || (a.kb == 2 && a.pad))
    return hipErrorInvalidValue;
  uint32_t grid;
  hipError_t e = grid_of(a.rows, a.lines, &grid);
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)a.lines * rader_line((uint32_t)a.n, a.pad != 0) * sizeof(float2);
  if (lds > (size_t)kLdsBudgetBytes) return hipErrorInvalidValue;
  const dim3 block((uint32_t)(a.tpl * a.lines));
  // block IO through LDS, as k_mixed does for short lines, here for every
  // p <= 4096 (the bound of its exact division).  Per 512 MiB: p = 5 906 ->
  // 170 us, 13 2962 -> 175, 17 4158 -> 318, 37 862 -> 326, 97 510 -> 335,
  // 257 720 -> 405, 641 481 -> 398; and with longer lines too, unlike
  // k_mixed: 1009 (144 threads per line) 600 -> 494, 2017 523 -> 459, 2593
  // 615 -> 537, 3001 747 -> 678, 4001 730 -> 701
  const bool stg = rd.p <= 4096;
  const size_t ldst = lds + (size_t)(a.n - a.radix[0]) * sizeof(float2);
  if (a.kb == 2)  // p - 1 above 8192: two butterflies of up to 16 values per thread
    FFTAMD_LAUNCH((k_rader<2, 16, false, false>), dim3(grid), block, lds, st, a, rd);
  else if (ldst <= (size_t)kLdsBudgetBytes && wg_per_cu(ldst, block.x) >= wg_per_cu(lds, block.x)) {
    if (a.pad && stg)
      FFTAMD_LAUNCH((k_rader<1, 16, true, true, true>), dim3(grid), block, ldst, st, a, rd);
    else if (a.pad)
      FFTAMD_LAUNCH((k_rader<1, 16, true, false, true>), dim3(grid), block, ldst, st, a, rd);
    else if (stg)
      FFTAMD_LAUNCH((k_rader<1, 16, false, true, true>), dim3(grid), block, ldst, st, a, rd);
    else
      FFTAMD_LAUNCH((k_rader<1, 16, false, false, true>), dim3(grid), block, ldst, st, a, rd);
  } else if (a.pad && stg)
    FFTAMD_LAUNCH((k_rader<1, 16, true, true>), dim3(grid), block, lds, st, a, rd);
  else if (a.pad)
    FFTAMD_LAUNCH((k_rader<1, 16, true, false>), dim3(grid), block, lds, st, a, rd);
  else if (stg)
    FFTAMD_LAUNCH((k_rader<1, 16, false, true>), dim3(grid), block, lds, st, a, rd);
  else
    FFTAMD_LAUNCH((k_rader<1, 16, false, false>), dim3(grid), block, lds, st, a, rd);
  return hipGetLastError();
}

hipError_t launch_bluestein_mixed(const MixedArgs& a, const ChirpMixedArgs& c, hipStream_t st) {
  int rmax = 0;
  if (!mixed_schedule_ok(a, &rmax) || a.kb != 1 || c.n < 2 || 2 * c.n - 1 > a.n || !a.pre || !c.bhat || !c.post)
    return hipErrorInvalidValue;
  uint32_t grid;
  hipError_t e = grid_of(a.rows, a.lines, &grid);
  if (e != hipSuccess) return e;
  const size_t lds =
      (size_t)a.lines * ((a.pad ? mixed_pad<true>((uint32_t)a.n) : mixed_pad<false>((uint32_t)a.n)) + 1) * sizeof(float2);
  if (lds > (size_t)kLdsBudgetBytes) return hipErrorInvalidValue;
  const dim3 block((uint32_t)(a.tpl * a.lines));
  // block IO through LDS for every row (n <= 4096 here): per 512 MiB 1034
  // 851 -> 755 us, 1049 816 -> 658, 2053 1119 -> 1049, 2111 1013 -> 972
  // beside the short-line gains (34 797 -> 473 with the mixed length)
  const bool stg = c.n <= 4096;
  const size_t ldst = lds + (size_t)(a.n - a.radix[0]) * sizeof(float2);
  if (ldst <= (size_t)kLdsBudgetBytes && wg_per_cu(ldst, block.x) >= wg_per_cu(lds, block.x)) {
    if (a.pad && stg)
      FFTAMD_LAUNCH((k_bluestein_mixed<true, true, true>), dim3(grid), block, ldst, st, a, c);
    else if (a.pad)
      FFTAMD_LAUNCH((k_bluestein_mixed<true, false, true>), dim3(grid), block, ldst, st, a, c);
    else if (stg)
      FFTAMD_LAUNCH((k_bluestein_mixed<false, true, true>), dim3(grid), block, ldst, st, a, c);
    else
      FFTAMD_LAUNCH((k_bluestein_mixed<false, false, true>), dim3(grid), block, ldst, st, a, c);
    return hipGetLastError();
  }
  if (a.pad && stg)
    FFTAMD_LAUNCH((k_bluestein_mixed<true, true>), dim3(grid), block, lds, st, a, c);
  else if (a.pad)
    FFTAMD_LAUNCH((k_bluestein_mixed<true, false>), dim3(grid), block, lds, st, a, c);
  else if (stg)
    FFTAMD_LAUNCH((k_bluestein_mixed<false, true>), dim3(grid), block, lds, st, a, c);
  else
    FFTAMD_LAUNCH((k_bluestein_mixed<false, false>), dim3(grid), block, lds, st, a, c);
  return hipGetLastError();
}

}  // namespace fftamd
