// Router: logits, softmax over all experts, top-k gates.
//
// "Dynamic Token Routing AI", "How it works": a gating network scores every token and the
// best-scoring experts are selected; Worked Example (trace of token 0): the chosen expert's
// output is later scaled by the router's confidence, here the softmax probability.
//
// Precision: the logits are sums of exact products (bf16*bf16 and fp32*fp32 products are
// exact in fp64) accumulated in fp64, the softmax is evaluated in fp64 and each probability
// is rounded once to fp32.  Top-k compares the fp32 gates, ties going to the lower expert.
// Slot assignment later orders tokens by these gates across the whole batch, so the gates
// have to be reproducible to the last fp32 bit: fp64 accumulation makes them independent of
// the summation order except in the rare case where a probability lies within fp64
// rounding noise of an fp32 rounding boundary.
//
// Mapping (gfx950): the logit GEMM is [T, d] x [d, E] with E <= 256, far too skinny for the
// matrix cores and bound by streaming x from HBM (or by the fp64 ALUs when E is large).
// Each lane owns one token; the S waves of a block split the columns.  The router weights,
// widened once to fp64, are read with wave-uniform addresses, so they arrive through the
// scalar cache into SGPRs and every lane does one fp64 FMA per (column, expert) with no
// cross-lane traffic; the S partial sums meet in LDS and are added in a fixed order.
#include "moe_internal.h"

namespace moe {

// Router weights widened to fp64 and laid out [group][d][EMAX] (experts g*EMAX .. g*EMAX +
// EMAX-1 of one column contiguous, zero-padded past E), so a column's weights are one aligned
// run of EMAX doubles: wide unconditional scalar loads.
template <typename TIn>
__global__ void k_router_weights_f64(const TIn* __restrict__ w, double* __restrict__ w64,
                                     int d, int E, int EMAX) {
  const int G = (E + EMAX - 1) / EMAX;
  const int64_t n = (int64_t)G * d * EMAX;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t g = i / ((int64_t)d * EMAX), rem = i % ((int64_t)d * EMAX);
    const int64_t j = rem / EMAX, e = g * EMAX + rem % EMAX;
    w64[i] = e < E ? (double)load_as_f32(w + e * d + j) : 0.0;
  }
}

template <typename TIn>
struct VecLoad;
template <>
struct VecLoad<bf16_t> {
  static constexpr int VW = 8;  // columns per 16-byte chunk
  __device__ __forceinline__ static uint4 raw(const bf16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
  }
  __device__ __forceinline__ static void widen(uint4 q, double* v) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (double)__uint_as_float(w[i] << 16);
      v[2 * i + 1] = (double)__uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct VecLoad<float> {
  static constexpr int VW = 4;
  __device__ __forceinline__ static uint4 raw(const float* p) {
    return *reinterpret_cast<const uint4*>(p);
  }
  __device__ __forceinline__ static void widen(uint4 q, double* v) {
    v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
    v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
  }
};

// Block: S waves x 64 lanes, 64 tokens (one per lane).  Wave s accumulates the partial
// logits of the block's tokens over the column chunks c = s (mod S); the chunk index is
// wave-uniform, so the fp64 router weights are read with uniform addresses (scalar loads).
template <int EMAX>
struct RouteBounds {
  // waves per block the partial-sum LDS allows (128 KiB / (EMAX * 64 lanes * 8 bytes)), <= 16
  static constexpr int kMaxS = (128 * 1024) / (EMAX * 64 * 8) < 16 ? (128 * 1024) / (EMAX * 64 * 8) : 16;
  static constexpr int kThreads = 64 * kMaxS;
};

template <typename TIn, int EMAX>
__global__ __launch_bounds__(RouteBounds<EMAX>::kThreads) void k_route(
    const TIn* __restrict__ x, const double* __restrict__ w64, const float* __restrict__ b_router,
    int64_t T, int d, int E, int k, int S, int32_t* __restrict__ ids,
    float* __restrict__ gates, float* __restrict__ logits_out) {
  extern __shared__ double lds[];  // partials [S][EMAX][64]; then logits/gates [E][64]
  constexpr int VW = VecLoad<TIn>::VW;
  constexpr int TB = 64;
  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; readfirstlane tells the compiler, so addresses built from
  // it (the router weights) are scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t tok0 = (int64_t)blockIdx.x * TB;
  const int64_t t = tok0 + lane;
  const bool tok_ok = t < T;
  const int n_groups = (E + EMAX - 1) / EMAX;  // > 1 only when S == 1 (host guarantees)
  const TIn* xrow = x + (tok_ok ? t : 0) * (int64_t)d;

  for (int g = 0; g < n_groups; ++g) {
    const int e0 = g * EMAX;
    const int eg = min(EMAX, E - e0);
    const double* wg = w64 + (int64_t)g * d * EMAX;  // this group's [d][EMAX] weights
    double acc[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[e] = 0.0;

    if (d % VW == 0) {
      // chunks c = wave, wave + S, ...; four chunk loads in flight before their FMAs
      constexpr int PF = 4;
      const int nchunk = d / VW;
      int c = wave;
      for (; c + (PF - 1) * S < nchunk; c += PF * S) {
        uint4 q[PF];
#pragma unroll
        for (int u = 0; u < PF; ++u)
          q[u] = tok_ok ? VecLoad<TIn>::raw(xrow + (int64_t)(c + u * S) * VW) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          double xv[VW];
          VecLoad<TIn>::widen(q[u], xv);
#pragma unroll
          for (int v = 0; v < VW; ++v) {
            const double* wc = wg + ((int64_t)(c + u * S) * VW + v) * EMAX;
#pragma unroll
            for (int e = 0; e < EMAX; ++e) acc[e] = fma(xv[v], wc[e], acc[e]);
          }
        }
      }
      for (; c < nchunk; c += S) {
        double xv[VW];
        VecLoad<TIn>::widen(tok_ok ? VecLoad<TIn>::raw(xrow + (int64_t)c * VW) : make_uint4(0, 0, 0, 0), xv);
#pragma unroll
        for (int v = 0; v < VW; ++v) {
          const double* wc = wg + ((int64_t)c * VW + v) * EMAX;
#pragma unroll
          for (int e = 0; e < EMAX; ++e) acc[e] = fma(xv[v], wc[e], acc[e]);
        }
      }
    } else {
      // generic column loop for widths that are not a multiple of the vector size
      for (int j = wave; j < d; j += S) {
        const double xv = tok_ok ? (double)load_as_f32(xrow + j) : 0.0;
#pragma unroll
        for (int e = 0; e < EMAX; ++e) acc[e] = fma(xv, wg[(int64_t)j * EMAX + e], acc[e]);
      }
    }

    if (S == 1) {
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if (e < eg) lds[(e0 + e) * TB + lane] = acc[e];
    } else {
#pragma unroll
      for (int e = 0; e < EMAX; ++e) lds[(wave * EMAX + e) * TB + lane] = acc[e];
    }
  }
  __syncthreads();

  // sum the S wave partials in order; the result lands where partial 0 was (the thread
  // that writes lds[e][i] is the only one reading partial 0 of (e, i))
  const int nthr = 64 * S;
  if (S > 1) {
    for (int p = threadIdx.x; p < E * TB; p += nthr) {
      const int e = p / TB, i = p % TB;
      double s = 0.0;
      for (int w = 0; w < S; ++w) s += lds[(w * EMAX + e) * TB + i];
      lds[e * TB + i] = s;
    }
    __syncthreads();
  }
  // bias (added once to the complete sum) and the optional fp32 logits
  for (int p = threadIdx.x; p < E * TB; p += nthr) {
    const int e = p / TB, i = p % TB;
    double L = lds[e * TB + i];
    if (b_router) L += (double)b_router[e];
    lds[e * TB + i] = L;
    if (logits_out && tok0 + i < T) logits_out[(tok0 + i) * E + e] = (float)L;
  }
  __syncthreads();

  // softmax + top-k: LPT = S lanes per token (a power of two <= 16, inside one wave);
  // lane `sub` owns experts e = sub (mod LPT)
  const int LPT = S;
  const int ti = threadIdx.x / LPT, sub = threadIdx.x % LPT;
  const int64_t tt = tok0 + ti;

  double m = -INFINITY;
  for (int e = sub; e < E; e += LPT) m = fmax(m, lds[e * TB + ti]);
  for (int off = LPT >> 1; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
  double z = 0.0;
  for (int e = sub; e < E; e += LPT) {
    const double v = exp(lds[e * TB + ti] - m);
    lds[e * TB + ti] = v;
    z += v;
  }
  for (int off = LPT >> 1; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
  for (int e = sub; e < E; e += LPT) lds[e * TB + ti] = (double)(float)(lds[e * TB + ti] / z);

  // k rounds of a group arg-max on (gate descending, expert ascending); gates are >= 0,
  // so their fp32 bit patterns order like their values; a taken expert is marked -1
  for (int c = 0; c < k; ++c) {
    unsigned long long best = 0;
    for (int e = sub; e < E; e += LPT) {
      const double gv = lds[e * TB + ti];
      if (gv < 0.0) continue;
      const unsigned long long key =
          ((unsigned long long)__float_as_uint((float)gv) << 32) | (0xFFFFFFFFull - (unsigned)e);
      best = key > best ? key : best;
    }
    for (int off = LPT >> 1; off >= 1; off >>= 1) {
      const unsigned long long o = __shfl_xor(best, off, 64);
      best = o > best ? o : best;
    }
    const int ew = (int)(0xFFFFFFFFull - (best & 0xFFFFFFFFull));
    if (ew % LPT == sub) lds[ew * TB + ti] = -1.0;
    if (sub == 0 && tt < T) {
      ids[tt * k + c] = ew;
      gates[tt * k + c] = __uint_as_float((uint32_t)(best >> 32));
    }
  }
}

namespace {
template <typename TIn, int EMAX>
hipError_t route_impl(const moe_shape& s, const TIn* x, const float* b_router, int32_t* ids,
                      float* gates, float* logits, const double* w64, hipStream_t st) {
  constexpr int VW = VecLoad<TIn>::VW;
  const int64_t T = s.T;
  const int d = s.d_model, E = s.n_experts;
  const int ncol = (d % VW == 0) ? d / VW : d;
  // S waves split the columns; partials take S * EMAX * 64 doubles of LDS
  int S = 1;
  if (E <= EMAX)
    while (2 * S <= RouteBounds<EMAX>::kMaxS && 2 * S <= ncol) S *= 2;
  const size_t lds = (size_t)8 * 64 * (S > 1 ? (size_t)S * EMAX : (size_t)E);
  static bool attr_set = false;  // allow up to 128 KiB of dynamic LDS, once per instantiation
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)k_route<TIn, EMAX>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const int64_t grid = (T + 63) / 64;
  hipLaunchKernelGGL((k_route<TIn, EMAX>), dim3((unsigned)grid), dim3(64 * S), lds, st, x, w64,
                     b_router, T, d, E, s.top_k, S, ids, gates, logits);
  return hipGetLastError();
}
}  // namespace

int route_emax(int E) { return E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : 64; }

hipError_t launch_route(const moe_shape& s, const void* x, const void* w_router,
                        const float* b_router, int32_t* ids, float* gates, float* logits,
                        double* w64, hipStream_t st) {
  const int64_t nw = (int64_t)(s.n_experts + route_emax(s.n_experts) - 1) / route_emax(s.n_experts) *
                    route_emax(s.n_experts) * s.d_model;
  const int cblocks = (int)((nw + 255) / 256 < 1024 ? (nw + 255) / 256 : 1024);
  const int E = s.n_experts, d = s.d_model;
  if (s.dtype == MOE_BF16) {
    hipLaunchKernelGGL(k_router_weights_f64<bf16_t>, dim3(cblocks), dim3(256), 0, st,
                       (const bf16_t*)w_router, w64, d, E, route_emax(E));
    const bf16_t* xp = (const bf16_t*)x;
    if (E <= 8) return route_impl<bf16_t, 8>(s, xp, b_router, ids, gates, logits, w64, st);
    if (E <= 16) return route_impl<bf16_t, 16>(s, xp, b_router, ids, gates, logits, w64, st);
    if (E <= 32) return route_impl<bf16_t, 32>(s, xp, b_router, ids, gates, logits, w64, st);
    return route_impl<bf16_t, 64>(s, xp, b_router, ids, gates, logits, w64, st);
  } else {
    hipLaunchKernelGGL(k_router_weights_f64<float>, dim3(cblocks), dim3(256), 0, st,
                       (const float*)w_router, w64, d, E, route_emax(E));
    const float* xp = (const float*)x;
    if (E <= 8) return route_impl<float, 8>(s, xp, b_router, ids, gates, logits, w64, st);
    if (E <= 16) return route_impl<float, 16>(s, xp, b_router, ids, gates, logits, w64, st);
    if (E <= 32) return route_impl<float, 32>(s, xp, b_router, ids, gates, logits, w64, st);
    return route_impl<float, 64>(s, xp, b_router, ids, gates, logits, w64, st);
  }
}

}  // namespace moe
