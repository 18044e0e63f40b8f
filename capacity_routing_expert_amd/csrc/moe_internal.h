// Internal declarations shared by the HIP sources of libmoe (not part of the C interface).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <atomic>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------- host helpers
constexpr int kMaxDevices = 64;

// Lets kernel `kern` take `bytes` of dynamic LDS on the current device, once per device:
// `done` is the kernel's own per-device flag array (a function-local static, zero at start).
// Concurrent first calls may both set the attribute, which is harmless.
inline hipError_t allow_dynamic_lds(const void* kern, int bytes,
                                    std::atomic<bool> (&done)[kMaxDevices]) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  err = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (err == hipSuccess && cached) done[dev].store(true, std::memory_order_release);
  return err;
}

typedef uint16_t bf16_t;  // bf16 stored as its bit pattern

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// round to nearest, ties to even (inputs here are finite)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}
// two floats to a packed bf16 pair (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b16x2_t));
}
// Buffer resource over `bytes` bytes at `base` (wave-uniform): a load at a byte offset at or past
// `bytes` (kBufferOOR, for one) reads zeros, so guarded loads need no branch.
constexpr uint32_t kBufferOOR = 0xFFFFFFF0u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ float load_as_f32(const bf16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load_as_f32(const float* p) { return *p; }

// 32-bit DPP lane move within rows of 16 lanes (all rows and banks enabled)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  return ((uint64_t)dpp32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp32<CTRL>((uint32_t)v);
}
// The value of lane (lane ^ stride), stride < 64.  Strides 1 and 2 are quad permutations and 8 a
// rotation by half a row, all DPP moves; stride 4 takes the rotations by 12 and by 4 (lane
// i reads lane i + 4 or i - 4 of its row) and keeps the one that lands on the partner; 16 and 32
// go through ds_bpermute.
__device__ __forceinline__ uint64_t xor_partner(uint64_t v, int stride) {
  switch (stride) {
    case 1: return dpp64<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    case 2: return dpp64<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    case 4: {
      const uint64_t up = dpp64<0x12C>(v), down = dpp64<0x124>(v);  // row_ror 12, row_ror 4
      return (threadIdx.x & 4) ? down : up;
    }
    case 8: return dpp64<0x128>(v);  // row_ror 8
    default: return __shfl_xor(v, stride, 64);
  }
}

// ---------------------------------------------------------------- workspace layout
// One workspace buffer serves every call; each sub-buffer starts on a 256-byte boundary.
struct Workspace {
  size_t ids;        // top-k expert ids (layer_forward)          [T*k] int32
  size_t gates;      // top-k gates                               [T*k] f32
  size_t slot_of;    // slot per assignment                       [T*k] int32
  size_t drop;       // drop mask                                 [T*k] u8
  size_t counts;     // per-expert assignment counts              [E] int32
  size_t offsets;    // kept-slot offsets                         [E+1] int32
  size_t seg_start;  // start of each expert's bucket in `keys`   [E+2] int32
  size_t blk_hist;   // per-block expert histograms               [nb, E+1] int32
  size_t keys;       // bucketed sort keys                        [T*k] u64
  size_t rank;       // rank of each bucketed key in its expert   [T*k] int32
  size_t row_token;  // token per slot (dropless: per sorted pair) [max_rows] int32
  size_t pairs;      // dropless: pairs sorted by expert          [T*k] int32 (else 0 B)
  size_t row_token_pad;  // padded layout: token per buffer row  [E * cap] int32 (else 0 B)
  size_t offsets_pad;    // padded layout: e * cap                   [E+1] int32 (else 0 B)
  size_t h;          // activation between the GEMMs              [rows, d_ff]
  size_t y;          // expert outputs per slot                   [rows, d_model]
                     // rows = max_rows (compact), E * cap (padded) or T * k (dropless, in
                     // pair order; the slot-dispatch buffers are then 0 B)
  size_t total;
};

constexpr int kDispatchChunk = 2048;  // most assignments per block in the count/scatter kernels
// Assignments per block of the count/scatter kernels for n assignments: a multiple of 256 near
// n / 32, from 256 up to kDispatchChunk.  pairs: the pair dispatch, which runs as one block up
// to kDispatchChunk assignments.
int dispatch_chunk(int64_t n, bool pairs = false);
int64_t dispatch_blocks(int64_t n, bool pairs = false);
// Runs of the two-launch dispatch for n assignments (0 where n takes another path); the
// blk_hist buffer holds runs * (E + 1) expert starts there.
int64_t dispatch_runs(int64_t n);

int64_t max_rows(const moe_shape& s);
enum LayoutKind { kLayoutCompact = 0, kLayoutPadded = 1, kLayoutDropless = 2 };
Workspace layout(const moe_shape& s, LayoutKind kind = kLayoutCompact);

// ---------------------------------------------------------------- launchers (return hipError_t)
hipError_t launch_route(const moe_shape& s, const void* x, const void* w_router,
                        const float* b_router, int32_t* ids, float* gates, float* logits,
                        hipStream_t st);

hipError_t launch_dispatch(const moe_shape& s, const int32_t* ids, const float* gates,
                           int32_t* counts, int32_t* offsets, int32_t* slot_of,
                           int32_t* row_token, uint8_t* drop, int32_t* seg_start,
                           int32_t* blk_hist, uint64_t* keys, int32_t* rank, hipStream_t st);

// x_routed[s] = x[row_token[s]] for the kept slots s < offsets[E] (rows of d_model elements of
// the shape's dtype); the grid covers max_rows(s) slots
hipError_t launch_gather_rows(const moe_shape& s, const void* x, const int32_t* row_token,
                              const int32_t* offsets, void* x_routed, hipStream_t st);

// Kernel timing: arm_launch_events(start, stop) makes the next timed launch on this thread (an
// expert GEMM, the router or the combine) record its own start and stop in the two events
// (hipExtLaunchKernel, no marker between launches); take_launch_events hands them to that
// launch and disarms.
void arm_launch_events(hipEvent_t start, hipEvent_t stop);
bool take_launch_events(hipEvent_t* start, hipEvent_t* stop);

// One kernel launch that takes the armed events, if any.
template <typename Kernel, typename... Args>
hipError_t launch_timed(Kernel kern, dim3 grid, dim3 block, size_t lds, hipStream_t st,
                        Args... args) {
  hipEvent_t t0, t1;
  if (take_launch_events(&t0, &t1))
    hipExtLaunchKernelGGL(kern, grid, block, lds, st, t0, t1, 0, args...);
  else
    hipLaunchKernelGGL(kern, grid, block, lds, st, args...);
  return hipGetLastError();
}

// rows_ub: an upper bound on the slot rows of the layout (max_rows(s) compact, E * capacity
// padded); row_token entries < 0 are zero rows
hipError_t launch_ffn_up(const moe_shape& s, const void* x, const int32_t* row_token,
                         const int32_t* offsets, const void* w1, const void* b1, void* h,
                         int64_t rows_ub, hipStream_t st);
hipError_t launch_ffn_down(const moe_shape& s, const void* h, const int32_t* offsets,
                           const void* w2, const void* b2, void* y, int64_t rows_ub,
                           hipStream_t st);

// gated expert: H = SiLU(x W_gate^T) * (x W_up^T) with W13 [E, 2 d_ff, d_model] (gate rows
// first), then Y = H W2^T; no biases; bf16 only
hipError_t launch_ffn_up_gated(const moe_shape& s, const void* x, const int32_t* row_token,
                               const int32_t* offsets, const void* w13, void* h, int64_t rows_ub,
                               hipStream_t st);
hipError_t launch_ffn_down_nobias(const moe_shape& s, const void* h, const int32_t* offsets,
                                  const void* w2, void* y, int64_t rows_ub, hipStream_t st);

// compact slots -> padded fixed buffers: slot_of (in place) becomes e * cap + rank, the padded
// row tokens (-1 for unused rows) and the padded offsets e * cap are written
hipError_t launch_pad_layout(const moe_shape& s, const int32_t* ids, const int32_t* offsets,
                             const int32_t* row_token, int32_t* slot_of, int32_t* row_token_pad,
                             int32_t* offsets_pad, hipStream_t st);

hipError_t launch_combine(const moe_shape& s, const void* x, const float* gates,
                          const int32_t* slot_of, const void* y, void* out, hipStream_t st);

// ---- dropless pair-order flow (bf16 GEMMs; moe_sum also fp32)
// pairs p = t*k + c grouped by expert, ascending p inside an expert; row_token = pair / k
hipError_t launch_dispatch_pairs(const moe_shape& s, const int32_t* ids, int32_t* counts,
                                 int32_t* offsets, int32_t* sorted_pairs, int32_t* row_token,
                                 int32_t* blk_hist, hipStream_t st);
// H[pair] = act(x[pair / k] W1^T (+ b1)); gated: W1 is W13 [E, 2 d_ff, d_model], no bias
hipError_t launch_ffn_up_pairs(const moe_shape& s, const void* x, const int32_t* row_token,
                               const int32_t* sorted_pairs, const int32_t* offsets,
                               const void* w1, const void* b1, void* h, int64_t rows_ub,
                               bool gated, hipStream_t st);
// Y[pair] = weights[pair] * (H[pair] W2^T (+ b2)); b2 may be NULL
hipError_t launch_ffn_down_pairs(const moe_shape& s, const void* h, const int32_t* sorted_pairs,
                                 const int32_t* offsets, const void* w2, const void* b2,
                                 const float* weights, void* y, int64_t rows_ub, hipStream_t st);
// out[t] = (x[t] +) sum of pair rows t*k .. t*k + k - 1 whose id is in [0, E) (all if ids NULL)
hipError_t launch_moe_sum(const moe_shape& s, const void* x, const int32_t* ids,
                          const void* rows, void* out, hipStream_t st);

// ---- packed expert weights: [E, rows, cols] -> [E, ceil(cols / 32), rows, 32]
int64_t packed_weight_elems(int64_t E, int rows, int cols);
hipError_t launch_pack_weights(const void* w, void* wp, int64_t E, int rows, int cols,
                               hipStream_t st);

// ---- batch consolidation
constexpr int kSchedMaxT = 8192;     // tokens one scheduling workgroup sorts (64 KiB of keys)
constexpr int kSchedIndexBits = 13;  // token index bits of a sort key
constexpr int kSchedMaxK = 8;
int schedule_bits_e(int E);          // bits of an expert id in a sort key (values 0 .. E)
// order[i] = token at position i: tokens sorted by expert set (ascending ids as a tuple), then
// by token index; T <= kSchedMaxT, k * schedule_bits_e(E) + kSchedIndexBits <= 64
hipError_t launch_schedule(const int32_t* ids, int T, int k, int E, int32_t* order,
                           hipStream_t st);
// out[b] = distinct experts in [0, E) of the tokens at positions b * B .. b * B + B - 1: token
// order[i] at position i, or token i when order is NULL (ids [M * B, k])
hipError_t launch_batch_experts(const int32_t* ids, const int32_t* order, int B, int M, int k,
                                int E, int32_t* out, hipStream_t st);
// rows of row_bytes (a multiple of 4): dst[i] = src[idx[i]], or dst[idx[i]] = src[i] (scatter)
hipError_t launch_permute_rows(const void* src, const int32_t* idx, void* dst, int64_t n,
                               int row_bytes, bool scatter, hipStream_t st);

}  // namespace moe
