// Expert FFN in fp32 (the fp32 dtype path): y = W2 SiLU(W1 x + b1) + b2 per kept slot.
//
// Worked Example, trace of token 0: up-projection with bias, SiLU element-wise,
// down-projection with bias.  A plain one-thread-per-output kernel pair with fp32
// accumulation in column order; it serves small fp32 layers such as the worked example,
// where the work is a few hundred FLOPs and latency is all that matters.
#include <hip/hip_ext.h>

#include "moe_internal.h"

namespace moe {

namespace {
// expert owning slot s: the e with offsets[e] <= s < offsets[e+1]
__device__ __forceinline__ int expert_of_slot(const int32_t* __restrict__ offsets, int E, int s) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= s) lo = mid; else hi = mid - 1;
  }
  return lo;
}
}  // namespace

__global__ __launch_bounds__(256) void k_ffn_up_f32(const float* __restrict__ x,
                                                    const int32_t* __restrict__ row_token,
                                                    const int32_t* __restrict__ offsets, int E,
                                                    const float* __restrict__ w1,
                                                    const float* __restrict__ b1,
                                                    float* __restrict__ h, int d, int f,
                                                    int64_t max_rows) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= max_rows * f) return;
  const int s = (int)(id / f), n = (int)(id % f);
  if (s >= offsets[E]) return;
  const int e = expert_of_slot(offsets, E, s);
  const int rt = row_token[s];  // -1: a zero row (padding)
  const float* wr = w1 + ((int64_t)e * f + n) * d;
  float acc = b1[(int64_t)e * f + n];
  if (rt >= 0) {
    const float* xr = x + (int64_t)rt * d;
    for (int j = 0; j < d; ++j) acc = fmaf(xr[j], wr[j], acc);
  }
  h[(int64_t)s * f + n] = acc / (1.0f + expf(-acc));
}

__global__ __launch_bounds__(256) void k_ffn_down_f32(const float* __restrict__ h,
                                                      const int32_t* __restrict__ offsets, int E,
                                                      const float* __restrict__ w2,
                                                      const float* __restrict__ b2,
                                                      float* __restrict__ y, int d, int f,
                                                      int64_t max_rows) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= max_rows * d) return;
  const int s = (int)(id / d), o = (int)(id % d);
  if (s >= offsets[E]) return;
  const int e = expert_of_slot(offsets, E, s);
  const float* hr = h + (int64_t)s * f;
  const float* wr = w2 + ((int64_t)e * d + o) * f;
  float acc = b2[(int64_t)e * d + o];
  for (int j = 0; j < f; ++j) acc = fmaf(hr[j], wr[j], acc);
  y[(int64_t)s * d + o] = acc;
}

hipError_t launch_ffn_up_f32(const moe_shape& s, const void* x, const int32_t* row_token,
                             const int32_t* offsets, const void* w1, const void* b1, void* h,
                             int64_t rows, hipStream_t st) {
  const int64_t n = rows * s.d_ff;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  hipEvent_t t0, t1;
  if (take_launch_events(&t0, &t1))
    hipExtLaunchKernelGGL(k_ffn_up_f32, grid, dim3(256), 0, st, t0, t1, 0, (const float*)x,
                          row_token, offsets, s.n_experts, (const float*)w1, (const float*)b1,
                          (float*)h, s.d_model, s.d_ff, rows);
  else
    hipLaunchKernelGGL(k_ffn_up_f32, grid, dim3(256), 0, st, (const float*)x, row_token, offsets,
                       s.n_experts, (const float*)w1, (const float*)b1, (float*)h, s.d_model,
                       s.d_ff, rows);
  return hipGetLastError();
}

hipError_t launch_ffn_down_f32(const moe_shape& s, const void* h, const int32_t* offsets,
                               const void* w2, const void* b2, void* y, int64_t rows,
                               hipStream_t st) {
  const int64_t n = rows * s.d_model;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  hipEvent_t t0, t1;
  if (take_launch_events(&t0, &t1))
    hipExtLaunchKernelGGL(k_ffn_down_f32, grid, dim3(256), 0, st, t0, t1, 0, (const float*)h,
                          offsets, s.n_experts, (const float*)w2, (const float*)b2, (float*)y,
                          s.d_model, s.d_ff, rows);
  else
    hipLaunchKernelGGL(k_ffn_down_f32, grid, dim3(256), 0, st, (const float*)h, offsets,
                       s.n_experts, (const float*)w2, (const float*)b2, (float*)y, s.d_model,
                       s.d_ff, rows);
  return hipGetLastError();
}

}  // namespace moe
