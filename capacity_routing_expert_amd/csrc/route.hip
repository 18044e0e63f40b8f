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
// Each lane owns one token; the P blocks of a token group and the S waves of a block split
// the columns, and each lane keeps up to 16 chunk loads of its row in flight.  The router
// weights, widened once to fp64, are read with wave-uniform addresses, so they arrive through
// the scalar cache into SGPRs and every lane does one fp64 FMA per (column, expert) with no
// cross-lane traffic; partial sums are added in a fixed order, so the logits do not depend on
// which block finishes first.
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
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = tid; i < n; i += (int64_t)gridDim.x * blockDim.x) {
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

template <int EMAX>
struct RouteBounds {
  // waves per block the partial-sum LDS allows (128 KiB / (EMAX * 64 lanes * 8 bytes)), <= 4
  static constexpr int kMaxS = (128 * 1024) / (EMAX * 64 * 8) < 4 ? (128 * 1024) / (EMAX * 64 * 8) : 4;
  static constexpr int kThreads = 64 * kMaxS;
};

constexpr int kRoutePF = 8;  // x chunks (one 128-byte line) a lane has in flight at once

// Bias, optional fp32 logits, softmax over all experts in fp64 (rounded once to fp32) and
// top-k for the 64 tokens whose complete logits sit in lds[e * 64 + i]; every thread of the
// block calls it (S lanes per token).
template <int TB>
__device__ void finish_group(double* lds, const float* __restrict__ b_router, int64_t tok0,
                             int64_t T, int E, int k, int S, int nthr, int32_t* __restrict__ ids,
                             float* __restrict__ gates, float* __restrict__ logits_out) {
  // bias (added once to the complete sum) and the optional fp32 logits
  for (int q = threadIdx.x; q < E * TB; q += nthr) {
    const int e = q / TB, i = q % TB;
    double L = lds[e * TB + i];
    if (b_router) L += (double)b_router[e];
    lds[e * TB + i] = L;
    if (logits_out && tok0 + i < T) logits_out[(tok0 + i) * E + e] = (float)L;
  }
  __syncthreads();

  // softmax + top-k: LPT = S lanes per token (a power of two <= 4, inside one wave);
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

// Block (g, p): 64 tokens (one per lane) of token group g, column partition p of P, split
// over the S waves of the block (wave s takes the s-th contiguous run of chunks).  The S
// wave partials meet in LDS in a fixed order.  With P > 1 the block writes its partial logits
// to `part`, and the last block of the group to arrive (an integer arrival counter) adds the
// P partials in partition order and finishes the token group; the result does not depend on
// which block arrives last.
template <typename TIn, int EMAX>
__global__ __launch_bounds__(RouteBounds<EMAX>::kThreads) void k_route(
    const TIn* __restrict__ x, const double* __restrict__ w64, const float* __restrict__ b_router,
    int64_t T, int d, int E, int k, int S, int P, double* __restrict__ part,
    int32_t* __restrict__ ids, float* __restrict__ gates, float* __restrict__ logits_out) {
  extern __shared__ double lds[];  // partials [S][EMAX][64]; then logits/gates [E][64]
  constexpr int VW = VecLoad<TIn>::VW;
  constexpr int TB = 64;
  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; readfirstlane tells the compiler, so addresses built from
  // it (the router weights) are scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = blockIdx.x / P, p = blockIdx.x % P;
  const int64_t tok0 = (int64_t)grp * TB;
  const int64_t t = tok0 + lane;
  const bool tok_ok = t < T;
  const int n_groups = (E + EMAX - 1) / EMAX;  // > 1 only when S == 1 and P == 1 (host)
  const TIn* xrow = x + (tok_ok ? t : 0) * (int64_t)d;
  const bool vec = d % VW == 0;
  const int ncol = vec ? d / VW : d;  // chunks (vector path) or columns
  const int cb = (int)((int64_t)ncol * p / P), ce = (int)((int64_t)ncol * (p + 1) / P);

  for (int g = 0; g < n_groups; ++g) {
    const int e0 = g * EMAX;
    const int eg = min(EMAX, E - e0);
    const double* wg = w64 + (int64_t)g * d * EMAX;  // this group's [d][EMAX] weights
    double acc[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[e] = 0.0;

    if (vec) {
      // this wave's chunks: a contiguous run of the partition, so each lane reads whole
      // 128-byte lines of its row; kRoutePF chunk loads in flight at a time
      const int per = (ce - cb + S - 1) / S;
      const int wb = cb + wave * per, we = min(ce, wb + per);
      for (int c0 = wb; c0 < we; c0 += kRoutePF) {
        uint4 q[kRoutePF];
#pragma unroll
        for (int u = 0; u < kRoutePF; ++u) {
          const int c = c0 + u;
          q[u] = (tok_ok && c < we) ? VecLoad<TIn>::raw(xrow + (int64_t)c * VW) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kRoutePF; ++u) {
          const int c = c0 + u;
          if (c >= we) break;  // wave-uniform
          double xv[VW];
          VecLoad<TIn>::widen(q[u], xv);
#pragma unroll
          for (int v = 0; v < VW; ++v) {
            const double* wc = wg + ((int64_t)c * VW + v) * EMAX;
#pragma unroll
            for (int e = 0; e < EMAX; ++e) acc[e] = fma(xv[v], wc[e], acc[e]);
          }
        }
      }
    } else {
      // generic column loop for widths that are not a multiple of the vector size
      for (int j = cb + wave; j < ce; j += S) {
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
    for (int q = threadIdx.x; q < E * TB; q += nthr) {
      const int e = q / TB, i = q % TB;
      double sum = 0.0;
      for (int w = 0; w < S; ++w) sum += lds[(w * EMAX + e) * TB + i];
      lds[e * TB + i] = sum;
    }
    __syncthreads();
  }

  if (P > 1) {
    // column partition p of the group: its partial logits go to `part`; k_route_finish adds
    // the P partials in partition order after this launch
    double* mine = part + ((int64_t)grp * P + p) * E * TB;
    for (int q = threadIdx.x; q < E * TB; q += nthr) mine[q] = lds[q];
    return;
  }
  finish_group<TB>(lds, b_router, tok0, T, E, k, S, nthr, ids, gates, logits_out);
}

// Token group g of 64: add the P partition partials in order, then bias, softmax, top-k.
template <int EMAXU>
__global__ __launch_bounds__(256) void k_route_finish(const double* __restrict__ part,
                                                      const float* __restrict__ b_router,
                                                      int64_t T, int E, int k, int P,
                                                      int32_t* __restrict__ ids,
                                                      float* __restrict__ gates,
                                                      float* __restrict__ logits_out) {
  extern __shared__ double lds[];  // [E][64]
  constexpr int TB = 64;
  const int64_t grp = blockIdx.x;
  const int S = blockDim.x / 64;
  for (int q = threadIdx.x; q < E * TB; q += blockDim.x) {
    // partials are loaded 8 at a time (independent loads) and added in partition order
    double sum = 0.0;
    for (int p0 = 0; p0 < P; p0 += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p0 + u < P ? part[(grp * P + p0 + u) * E * TB + q] : 0.0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (p0 + u < P) sum += v[u];
    }
    lds[q] = sum;
  }
  __syncthreads();
  finish_group<TB>(lds, b_router, grp * TB, T, E, k, S, (int)blockDim.x, ids, gates, logits_out);
}
int route_emax(int E) { return E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : 64; }

RoutePlan route_plan(const moe_shape& s) {
  RoutePlan r;
  const int E = s.n_experts, emax = route_emax(E);
  const int vw = s.dtype == MOE_BF16 ? 8 : 4;
  const int ncol = (s.d_model % vw == 0) ? s.d_model / vw : s.d_model;
  const int max_s = (128 * 1024) / (emax * 64 * 8) < 4 ? (128 * 1024) / (emax * 64 * 8) : 4;
  r.S = 1;
  if (E <= emax)
    while (2 * r.S <= max_s && 2 * r.S <= ncol) r.S *= 2;
  r.G = (s.T + 63) / 64;
  // enough waves to keep every SIMD streaming x (small E) or busy with fp64 FMAs (large E);
  // at least one column chunk per wave
  const int64_t target = E <= 16 ? 4096 : 1024;
  r.P = 1;
  if (E <= emax)
    while (r.P < 64 && r.G * r.P * r.S < target && (int64_t)2 * r.P * r.S <= ncol) r.P *= 2;
  return r;
}

namespace {

template <typename TIn, int EMAX>
hipError_t route_impl(const moe_shape& s, const TIn* x, const float* b_router, int32_t* ids,
                      float* gates, float* logits, const double* w64, double* part,
                      hipStream_t st) {
  const RoutePlan r = route_plan(s);
  const size_t lds = (size_t)8 * 64 * (r.S > 1 ? (size_t)r.S * EMAX : (size_t)s.n_experts);
  static bool attr_set = false;  // allow up to 128 KiB of dynamic LDS, once per instantiation
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)k_route<TIn, EMAX>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_route<TIn, EMAX>), dim3((unsigned)(r.G * r.P)), dim3(64 * r.S), lds, st,
                     x, w64, b_router, s.T, s.d_model, s.n_experts, s.top_k, r.S, r.P, part, ids,
                     gates, logits);
  if (r.P > 1) {
    const size_t lds2 = (size_t)8 * 64 * s.n_experts;
    hipLaunchKernelGGL((k_route_finish<EMAX>), dim3((unsigned)r.G), dim3(256), lds2, st, part,
                       b_router, s.T, s.n_experts, s.top_k, r.P, ids, gates, logits);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const moe_shape& s, const void* x, const void* w_router,
                        const float* b_router, int32_t* ids, float* gates, float* logits,
                        double* w64, double* part, hipStream_t st) {
  const int E = s.n_experts, d = s.d_model, emax = route_emax(E);
  const int64_t nw = (int64_t)(E + emax - 1) / emax * emax * d;
  const int cblocks = (int)((nw + 255) / 256 < 1024 ? (nw + 255) / 256 : 1024);
  if (s.dtype == MOE_BF16) {
    hipLaunchKernelGGL(k_router_weights_f64<bf16_t>, dim3(cblocks), dim3(256), 0, st,
                       (const bf16_t*)w_router, w64, d, E, emax);
    const bf16_t* xp = (const bf16_t*)x;
    if (E <= 8) return route_impl<bf16_t, 8>(s, xp, b_router, ids, gates, logits, w64, part, st);
    if (E <= 16) return route_impl<bf16_t, 16>(s, xp, b_router, ids, gates, logits, w64, part, st);
    if (E <= 32) return route_impl<bf16_t, 32>(s, xp, b_router, ids, gates, logits, w64, part, st);
    return route_impl<bf16_t, 64>(s, xp, b_router, ids, gates, logits, w64, part, st);
  } else {
    hipLaunchKernelGGL(k_router_weights_f64<float>, dim3(cblocks), dim3(256), 0, st,
                       (const float*)w_router, w64, d, E, emax);
    const float* xp = (const float*)x;
    if (E <= 8) return route_impl<float, 8>(s, xp, b_router, ids, gates, logits, w64, part, st);
    if (E <= 16) return route_impl<float, 16>(s, xp, b_router, ids, gates, logits, w64, part, st);
    if (E <= 32) return route_impl<float, 32>(s, xp, b_router, ids, gates, logits, w64, part, st);
    return route_impl<float, 64>(s, xp, b_router, ids, gates, logits, w64, part, st);
  }
}

}  // namespace moe
