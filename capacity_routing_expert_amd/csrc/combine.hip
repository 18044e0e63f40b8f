// Combine: gate-weighted expert outputs added to the residual.
//
// Worked Example, traces of tokens 0 and 4: a kept token leaves the layer as
// x + confidence * y, the dropped token as x itself.  With k > 1 the kept choices are summed
// in choice order, in fp32, with one rounding to the storage type at the end.  A token with
// no kept choice is copied bit for bit ("Some Tokens Do Not Get In", "Past the edge": it
// reaches the next layer exactly as it entered), so x + 0 never turns -0.0 into +0.0.
//
// HBM-bound stream: one wave per token row, 16-byte loads and streaming (nontemporal) stores;
// the row's x is requested first, then its slots and gates (one vector load of all choices),
// then the kept rows of Y.
#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ void widen8(uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void fma8(float g, uint4 v, float* acc) {
  float y[8];
  widen8(v, y);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, y[i], acc[i]);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at `base` (wave-uniform); loads past the range read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int ch) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, ch * 16, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16-byte streaming store (the output row is not read again by this layer)
__device__ __forceinline__ void store_nt(uint4 v, uint4* p) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

}  // namespace

// The kept choices of row t, in choice order: lane c of each 64-choice chunk loads slot and gate
// of choice c, so all of a row's choices arrive in one round trip; a ballot gives the kept ones.
// Returns the number kept and the first two (slot, gate) pairs (all wave-uniform).
__device__ __forceinline__ int kept_choices(const int32_t* __restrict__ slot_of,
                                            const float* __restrict__ gates, int64_t t, int k,
                                            int& s0, float& g0, int& s1, float& g1) {
  const int lane = threadIdx.x & 63;
  int n = 0;
  s0 = s1 = 0;
  g0 = g1 = 0.0f;
  for (int c0 = 0; c0 < k; c0 += 64) {
    const int m = min(64, k - c0);
    const __amdgpu_buffer_rsrc_t sr = row_rsrc(slot_of + t * k + c0, (uint32_t)m * 4u);
    const __amdgpu_buffer_rsrc_t gr = row_rsrc(gates + t * k + c0, (uint32_t)m * 4u);
    const int sl = lane < m ? (int)__builtin_amdgcn_raw_buffer_load_b32(sr, lane * 4, 0, 0) : -1;
    const float gl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(gr, lane * 4, 0, 0));
    uint64_t kept = __ballot(sl >= 0);
    while (kept && n < 2) {
      const int c = __builtin_amdgcn_readfirstlane(__ffsll((long long)kept) - 1);
      const int sc = __builtin_amdgcn_readlane(sl, c);
      const float gc = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(gl), c));
      if (n == 0) { s0 = sc; g0 = gc; } else { s1 = sc; g1 = gc; }
      ++n;
      kept &= kept - 1;
    }
    n += __popcll(kept);
  }
  return n;
}

// One wave per token row; each lane takes 16-byte chunks lane, lane + 64, ... in batches of
// kB.  The first batch of x is loaded before the row's slots are looked up (it depends on
// nothing); the y chunks of the first two kept choices follow as soon as the slots are known,
// so a row costs one memory round trip after the slot lookup per batch (plus one per further
// kept choice).
__global__ __launch_bounds__(256) void k_combine_bf16(const bf16_t* __restrict__ x,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ slot_of,
                                                      const bf16_t* __restrict__ y,
                                                      bf16_t* __restrict__ out, int64_t T, int d,
                                                      int k) {
  constexpr int kB = 4;
  const int lane = threadIdx.x & 63;
  // the row is wave-uniform; readfirstlane lets the compiler keep it, the slots, the gates and
  // the buffer resources in scalar registers
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;
  const int nch = d / 8;
  uint4* orow = reinterpret_cast<uint4*>(out + t * (int64_t)d);
  // rows as buffer ranges: chunks past the row, and the rows of absent choices, read as zeros
  const uint32_t row_bytes = (uint32_t)d * 2u;
  const __amdgpu_buffer_rsrc_t xb = row_rsrc(x + t * (int64_t)d, row_bytes);
  uint4 xv[kB];
#pragma unroll
  for (int b = 0; b < kB; ++b) xv[b] = load16(xb, lane + 64 * b);
  int s0, s1;
  float g0, g1;
  const int n_kept = kept_choices(slot_of, gates, t, k, s0, g0, s1, g1);
  const __amdgpu_buffer_rsrc_t y0 = row_rsrc(y + (int64_t)s0 * d, n_kept >= 1 ? row_bytes : 0u);
  const __amdgpu_buffer_rsrc_t y1 = row_rsrc(y + (int64_t)s1 * d, n_kept >= 2 ? row_bytes : 0u);

  for (int base = lane; base < nch; base += 64 * kB) {
    if (base != lane) {
#pragma unroll
      for (int b = 0; b < kB; ++b) xv[b] = load16(xb, base + 64 * b);
    }
    if (n_kept == 0) {  // every choice dropped: the row leaves bit for bit
#pragma unroll
      for (int b = 0; b < kB; ++b)
        if (base + 64 * b < nch) store_nt(xv[b], orow + base + 64 * b);
      continue;
    }
    uint4 v0[kB], v1[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      v0[b] = load16(y0, base + 64 * b);
      v1[b] = load16(y1, base + 64 * b);
    }
    float acc[kB][8];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      widen8(xv[b], acc[b]);
      fma8(g0, v0[b], acc[b]);
      if (n_kept >= 2) fma8(g1, v1[b], acc[b]);
    }
    if (n_kept > 2) {  // further kept choices, in choice order
      int seen = 0;
      for (int c = 0; c < k; ++c) {
        const int sc = slot_of[t * k + c];
        if (sc < 0 || ++seen <= 2) continue;
        const float g = gates[t * k + c];
        const __amdgpu_buffer_rsrc_t yc = row_rsrc(y + (int64_t)sc * d, row_bytes);
        uint4 vc[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) vc[b] = load16(yc, base + 64 * b);
#pragma unroll
        for (int b = 0; b < kB; ++b) fma8(g, vc[b], acc[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      if (base + 64 * b >= nch) continue;
      uint4 o;
      o.x = pack_bf16x2(acc[b][0], acc[b][1]);
      o.y = pack_bf16x2(acc[b][2], acc[b][3]);
      o.z = pack_bf16x2(acc[b][4], acc[b][5]);
      o.w = pack_bf16x2(acc[b][6], acc[b][7]);
      store_nt(o, orow + base + 64 * b);
    }
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

// ---------------------------------------------------------------- moe_sum
// moe_sum box of the fused-MoE flow diagram: pair order back to token order.  Token t leaves as
// the sum of its pair rows t*k .. t*k + k - 1 (GEMM 2 has already multiplied each by its top-k
// weight), plus the residual x[t] when one is given, summed in choice order in fp32 with one
// rounding.  With ids given, a pair whose expert id is outside [0, E) has no row and adds
// nothing; a token left with no row leaves as x[t] bit for bit (zeros without a residual).
// Same stream shape as the combine: one wave per token, 16-byte loads, streaming stores; the
// rows of a token are contiguous here, so no slot indirection.
__global__ __launch_bounds__(256) void k_moe_sum_bf16(const bf16_t* __restrict__ x,
                                                      const int32_t* __restrict__ ids,
                                                      const bf16_t* __restrict__ rows,
                                                      bf16_t* __restrict__ out, int64_t T, int d,
                                                      int k, int E) {
  constexpr int kB = 4;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;
  const int nch = d / 8;
  uint4* orow = reinterpret_cast<uint4*>(out + t * (int64_t)d);
  int n = 0, c0 = 0, c1 = 0;  // rows present, first two of them (wave-uniform)
  for (int c = 0; c < k; ++c) {
    if (ids && (uint32_t)ids[t * k + c] >= (uint32_t)E) continue;
    if (n == 0) c0 = c; else if (n == 1) c1 = c;
    ++n;
  }
  const uint32_t row_bytes = (uint32_t)d * 2u;
  const bf16_t* prow = rows + t * (int64_t)k * d;
  const __amdgpu_buffer_rsrc_t xb = row_rsrc(x ? x + t * (int64_t)d : rows, x ? row_bytes : 0u);
  const __amdgpu_buffer_rsrc_t y0 = row_rsrc(prow + (int64_t)c0 * d, n >= 1 ? row_bytes : 0u);
  const __amdgpu_buffer_rsrc_t y1 = row_rsrc(prow + (int64_t)c1 * d, n >= 2 ? row_bytes : 0u);
  for (int base = lane; base < nch; base += 64 * kB) {
    uint4 xv[kB], v0[kB], v1[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      xv[b] = load16(xb, base + 64 * b);
      v0[b] = load16(y0, base + 64 * b);
      v1[b] = load16(y1, base + 64 * b);
    }
    if (n == 0) {  // nothing to add: the residual (or zeros) bit for bit
#pragma unroll
      for (int b = 0; b < kB; ++b)
        if (base + 64 * b < nch) store_nt(xv[b], orow + base + 64 * b);
      continue;
    }
    float acc[kB][8];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      float y[8];
      widen8(xv[b], acc[b]);
      widen8(v0[b], y);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[b][i] += y[i];
      if (n >= 2) {
        widen8(v1[b], y);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[b][i] += y[i];
      }
    }
    if (n > 2) {  // further rows, in choice order
      int seen = 0;
      for (int c = 0; c < k; ++c) {
        if (ids && (uint32_t)ids[t * k + c] >= (uint32_t)E) continue;
        if (++seen <= 2) continue;
        const __amdgpu_buffer_rsrc_t yc = row_rsrc(prow + (int64_t)c * d, row_bytes);
        uint4 vc[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) vc[b] = load16(yc, base + 64 * b);
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          float y[8];
          widen8(vc[b], y);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[b][i] += y[i];
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      if (base + 64 * b >= nch) continue;
      uint4 o;
      o.x = pack_bf16x2(acc[b][0], acc[b][1]);
      o.y = pack_bf16x2(acc[b][2], acc[b][3]);
      o.z = pack_bf16x2(acc[b][4], acc[b][5]);
      o.w = pack_bf16x2(acc[b][6], acc[b][7]);
      store_nt(o, orow + base + 64 * b);
    }
  }
}

__global__ __launch_bounds__(256) void k_moe_sum_f32(const float* __restrict__ x,
                                                     const int32_t* __restrict__ ids,
                                                     const float* __restrict__ rows,
                                                     float* __restrict__ out, int64_t T, int d,
                                                     int k, int E) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float* orow = out + t * (int64_t)d;
  const float* prow = rows + t * (int64_t)k * d;
  for (int j = lane; j < d; j += 64) {
    float acc = x ? x[t * (int64_t)d + j] : 0.0f;
    for (int c = 0; c < k; ++c) {
      if (ids && (uint32_t)ids[t * k + c] >= (uint32_t)E) continue;
      acc += prow[(int64_t)c * d + j];
    }
    orow[j] = acc;
  }
}

hipError_t launch_moe_sum(const moe_shape& s, const void* x, const int32_t* ids,
                          const void* rows, void* out, hipStream_t st) {
  const int64_t grid = (s.T + 3) / 4;
  if (s.dtype == MOE_BF16)
    hipLaunchKernelGGL(k_moe_sum_bf16, dim3((unsigned)grid), dim3(256), 0, st, (const bf16_t*)x,
                       ids, (const bf16_t*)rows, (bf16_t*)out, s.T, s.d_model, s.top_k,
                       s.n_experts);
  else
    hipLaunchKernelGGL(k_moe_sum_f32, dim3((unsigned)grid), dim3(256), 0, st, (const float*)x,
                       ids, (const float*)rows, (float*)out, s.T, s.d_model, s.top_k,
                       s.n_experts);
  return hipGetLastError();
}

hipError_t launch_combine(const moe_shape& s, const void* x, const float* gates,
                          const int32_t* slot_of, const void* y, void* out, hipStream_t st) {
  const int64_t grid = (s.T + 3) / 4;
  if (s.dtype == MOE_BF16)
    return launch_timed(k_combine_bf16, dim3((unsigned)grid), dim3(256), 0, st, (const bf16_t*)x,
                        gates, slot_of, (const bf16_t*)y, (bf16_t*)out, s.T, s.d_model, s.top_k);
  return launch_timed(k_combine_f32, dim3((unsigned)grid), dim3(256), 0, st, (const float*)x,
                      gates, slot_of, (const float*)y, (float*)out, s.T, s.d_model, s.top_k);
}

}  // namespace moe
