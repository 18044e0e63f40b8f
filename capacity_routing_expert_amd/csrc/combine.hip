// Combine: gate-weighted expert outputs added to the residual.
//
// Worked Example, traces of tokens 0 and 4: a kept token leaves the layer as
// x + confidence * y, the dropped token as x itself.  With k > 1 the kept choices are summed
// in choice order, in fp32, with one rounding to the storage type at the end.  A token with
// no kept choice is copied bit for bit ("Some Tokens Do Not Get In", "Past the edge": it
// reaches the next layer exactly as it entered), so x + 0 never turns -0.0 into +0.0.
//
// HBM-bound stream: one wave per token row, 16-byte loads and stores; the slot numbers and
// gates of the row are wave-uniform (scalar loads).
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void k_combine_bf16(const bf16_t* __restrict__ x,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ slot_of,
                                                      const bf16_t* __restrict__ y,
                                                      bf16_t* __restrict__ out, int64_t T, int d,
                                                      int k) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nch = d / 8;
  const uint4* xr = reinterpret_cast<const uint4*>(x + t * (int64_t)d);
  uint4* orow = reinterpret_cast<uint4*>(out + t * (int64_t)d);
  bool any = false;
  for (int c = 0; c < k; ++c) any |= slot_of[t * k + c] >= 0;
  if (!any) {
    for (int ch = lane; ch < nch; ch += 64) orow[ch] = xr[ch];
    return;
  }
  for (int ch = lane; ch < nch; ch += 64) {
    const uint4 xv = xr[ch];
    float acc[8];
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = __uint_as_float(xw[i] << 16);
      acc[2 * i + 1] = __uint_as_float(xw[i] & 0xFFFF0000u);
    }
    for (int c = 0; c < k; ++c) {
      const int s = slot_of[t * k + c];
      if (s < 0) continue;
      const float g = gates[t * k + c];
      const uint4 yv = reinterpret_cast<const uint4*>(y + (int64_t)s * d)[ch];
      const uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(g, __uint_as_float(yw[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(g, __uint_as_float(yw[i] & 0xFFFF0000u), acc[2 * i + 1]);
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)f32_to_bf16(acc[2 * i]) | ((uint32_t)f32_to_bf16(acc[2 * i + 1]) << 16);
    orow[ch] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ __launch_bounds__(256) void k_combine_f32(const float* __restrict__ x,
                                                     const float* __restrict__ gates,
                                                     const int32_t* __restrict__ slot_of,
                                                     const float* __restrict__ y,
                                                     float* __restrict__ out, int64_t T, int d,
                                                     int k) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* xr = x + t * (int64_t)d;
  float* orow = out + t * (int64_t)d;
  bool any = false;
  for (int c = 0; c < k; ++c) any |= slot_of[t * k + c] >= 0;
  for (int j = lane; j < d; j += 64) {
    if (!any) {
      orow[j] = xr[j];
      continue;
    }
    float acc = xr[j];
    for (int c = 0; c < k; ++c) {
      const int s = slot_of[t * k + c];
      if (s < 0) continue;
      acc = fmaf(gates[t * k + c], y[(int64_t)s * d + j], acc);
    }
    orow[j] = acc;
  }
}

hipError_t launch_combine(const moe_shape& s, const void* x, const float* gates,
                          const int32_t* slot_of, const void* y, void* out, hipStream_t st) {
  const int64_t grid = (s.T + 3) / 4;
  if (s.dtype == MOE_BF16)
    hipLaunchKernelGGL(k_combine_bf16, dim3((unsigned)grid), dim3(256), 0, st, (const bf16_t*)x,
                       gates, slot_of, (const bf16_t*)y, (bf16_t*)out, s.T, s.d_model, s.top_k);
  else
    hipLaunchKernelGGL(k_combine_f32, dim3((unsigned)grid), dim3(256), 0, st, (const float*)x,
                       gates, slot_of, (const float*)y, (float*)out, s.T, s.d_model, s.top_k);
  return hipGetLastError();
}

}  // namespace moe
