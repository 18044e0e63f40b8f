// Expert FFN in bf16 on the matrix cores: two grouped GEMMs over the routed rows.
//
// Worked Example, trace of token 0: h = W1 x + b1, a = SiLU(h), y = W2 a + b2, each expert
// on its own batch of kept tokens; the closing paragraph of that page notes that the experts
// run side by side and the busiest one sets the wall-clock time.  Fused-MoE flow diagram
// (moe-vllm flow), boxes GEMM 1 and GEMM 2: the first GEMM reads its token rows through an
// index (the reorder happens on GEMM 1's read side) and each block works with one expert's
// weights.  Here the index is row_token[slot]; the rows stay in expert-slot order until the
// combine.
//
//   GEMM 1 (GATHER, SILU): H[s, n] = SiLU(sum_k x[row_token[s], k] W1[e, n, k] + b1[e, n])
//   GEMM 2               : Y[s, n] = sum_k H[s, k] W2[e, n, k] + b2[e, n]
// for every kept slot s of expert e.  Both operands are K-contiguous ("NT" GEMM), which is
// what v_mfma_f32_32x32x16_bf16 wants: each lane feeds 8 consecutive K values of one row.
//
// Tile: TN output features x TM slots x 64 K per stage; WN x WM waves, each owning a
// (TN/WN) x (TM/WM) sub-tile made of 32x32 MFMA blocks.  The weights play the MFMA "A" role
// and the token rows the "B" role, so a lane's accumulator holds 4 consecutive output
// features of one slot (8-byte stores).  Both operand tiles are staged through LDS with a
// 16-byte-chunk XOR swizzle (chunk c of row r lives at c ^ (r & 7)) so the MFMA fragment
// reads spread over the banks; the next stage's global loads are in flight while the current
// stage's MFMAs run (double-buffered LDS, one barrier per stage).  fp32 accumulation; bias,
// activation and the bf16 rounding happen in the epilogue.
//
// Scheduling: the grid is an upper bound (the number of kept rows is only known on the
// device).  Each block maps its index to (n-tile, m-tile), finds the expert of its m-tile
// from expert_offsets with a wave prefix scan, and exits if the tile does not exist.  Block
// indices are remapped so that consecutive logical tiles land on the same XCD (workgroups
// are dealt round-robin over the 8 XCDs), and logical tiles run m-tile-fastest within an
// n-tile: the blocks sharing an L2 share the weight tile and stream different token rows.
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

}  // namespace

template <int TN, int TM, int WN, int WM, bool GATHER, bool SILU>
__global__ __launch_bounds__(WN* WM * 64, 1) void k_grouped_gemm(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ W,
    const bf16_t* __restrict__ bias, bf16_t* __restrict__ out, int E, int N, int K, int mt_ub,
    int n_tiles) {
  constexpr int kThreads = WN * WM * 64;
  constexpr int FN = TN / WN / 32;
  constexpr int FM = TM / WM / 32;
  constexpr int kWPer = TN * 8 / kThreads;  // 16-byte chunks per thread per stage
  constexpr int kXPer = TM * 8 / kThreads;
  static_assert(kWPer * kThreads == TN * 8 && kXPer * kThreads == TM * 8, "tile/threads");
  extern __shared__ uint4 smem[];
  uint4* sW = smem;               // [2][TN][8] chunks
  uint4* sX = smem + 2 * TN * 8;  // [2][TM][8] chunks

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wm = wave / WN;

  const int G = gridDim.x;
  const int logical = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int nt = logical / mt_ub, mt = logical % mt_ub;
  if (nt >= n_tiles) return;

  // ---- expert of m-tile `mt` (lane L looks after experts 4L .. 4L+3)
  int e, row0, rows;
  {
    int te[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ee = lane * 4 + j;
      const int kept = ee < E ? offsets[ee + 1] - offsets[ee] : 0;
      te[j] = (kept + TM - 1) / TM;
      local += te[j];
    }
    int inc = local;
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(inc, off, 64);
      if (lane >= off) inc += o;
    }
    const int excl = inc - local;
    const int total = __builtin_amdgcn_readfirstlane(__shfl(inc, 63, 64));
    if (mt >= total) return;  // same decision in every wave of the block
    const uint64_t bal = __ballot(mt >= excl && mt < inc);
    const int owner = __ffsll((long long)bal) - 1;
    int esel = 0, tstart = 0, run = excl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (esel == 0 && mt >= run && mt < run + te[j]) {
        esel = lane * 4 + j + 1;
        tstart = run;
      }
      run += te[j];
    }
    // the same in every lane: make it scalar so the buffer resources live in SGPRs
    e = __builtin_amdgcn_readfirstlane(__shfl(esel, owner, 64) - 1);
    tstart = __builtin_amdgcn_readfirstlane(__shfl(tstart, owner, 64));
    row0 = offsets[e] + (mt - tstart) * TM;
    rows = min(TM, offsets[e + 1] - row0);
  }

  // ---- per-thread load plan.  Thread tid moves 16-byte chunk c = tid % 8 of rows
  // tid / 8 + r * kRowStep (r = 0 .. kWPer-1 / kXPer-1) of each operand tile.  Loads go through
  // buffer resources whose range covers only the valid rows: an out-of-range offset reads as
  // zero, so ragged tiles need no branches; chunks past K are sent out of range too.
  constexpr int kRowStep = kThreads / 8;
  const int c8 = (tid & 7) * 8;           // first K element of this thread's chunk
  const int trow = tid >> 3;              // first tile row of this thread
  const uint32_t kOut = 0x80000000u;      // an offset beyond every buffer range used here
  const int n0 = nt * TN;
  const int wrows = min(TN, N - n0);
  const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + ((int64_t)e * N + n0) * K), (short)0, wrows * K * 2, 0x00020000);
  const uint32_t woff = (uint32_t)(trow * K + c8) * 2u;
  const uint32_t wstep = (uint32_t)kRowStep * K * 2u;
  __amdgpu_buffer_rsrc_t xsrc;
  uint32_t xoff[kXPer];
  if (GATHER) {
    // x rows of the tile's tokens; the whole x is one resource (T * K * 2 < 2^31, checked on host)
    xsrc = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
    for (int r = 0; r < kXPer; ++r) {
      const int row = trow + r * kRowStep;
      xoff[r] = row < rows ? (uint32_t)(row_token[row0 + row] * K + c8) * 2u : kOut;
    }
  } else {
    xsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (int64_t)row0 * K), (short)0, rows * K * 2,
                                             0x00020000);
#pragma unroll
    for (int r = 0; r < kXPer; ++r) xoff[r] = (uint32_t)((trow + r * kRowStep) * K + c8) * 2u;
  }
  // LDS destinations: chunk c of row `row` lives at row * 8 + (c ^ (row & 7)); row & 7 is the
  // same for all r because kRowStep is a multiple of 8
  const int sdst = trow * 8 + ((tid & 7) ^ (trow & 7));

  uint4 rw[kWPer], rx[kXPer];

  f32x16_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (K + 63) / 64;
  const int r32 = lane & 31, half = lane >> 5;
  for (int kt = -1; kt < nk; ++kt) {
    // global loads of stage kt + 1 (in flight while stage kt computes)
    if (kt + 1 < nk) {
      const int k0 = (kt + 1) * 64;
      const bool kin = k0 + c8 < K;
      const uint32_t kb = (uint32_t)k0 * 2u;
#pragma unroll
      for (int r = 0; r < kWPer; ++r)
        rw[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    wsrc, kin ? woff + r * wstep + kb : kOut, 0, 0));
#pragma unroll
      for (int r = 0; r < kXPer; ++r)
        rx[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    xsrc, (kin && xoff[r] != kOut) ? xoff[r] + kb : kOut, 0, 0));
    }
    if (kt >= 0) {
      const int buf = kt & 1;
      const uint4* bw = sW + buf * TN * 8;
      const uint4* bx = sX + buf * TM * 8;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ch = kk * 2 + half;
        bf16x8_t a[FN], b[FM];
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int row = wn * (TN / WN) + i * 32 + r32;
          a[i] = as_bf16x8(bw[row * 8 + (ch ^ (row & 7))]);
        }
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int row = wm * (TM / WM) + j * 32 + r32;
          b[j] = as_bf16x8(bx[row * 8 + (ch ^ (row & 7))]);
        }
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int j = 0; j < FM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) {
      const int buf = (kt + 1) & 1;
#pragma unroll
      for (int r = 0; r < kWPer; ++r) sW[buf * TN * 8 + sdst + r * kRowStep * 8] = rw[r];
#pragma unroll
      for (int r = 0; r < kXPer; ++r) sX[buf * TM * 8 + sdst + r * kRowStep * 8] = rx[r];
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds features 8*(v/4) + 4*half + v%4 of slot column r32
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int tl = wm * (TM / WM) + j * 32 + r32;
    if (tl >= rows) continue;
    bf16_t* orow = out + (int64_t)(row0 + tl) * N;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = nt * TN + wn * (TN / WN) + i * 32 + 8 * g + 4 * half;
        if (n >= N) continue;
        const uint2 bb = *reinterpret_cast<const uint2*>(bias + (int64_t)e * N + n);
        float v[4];
        v[0] = acc[i][j][4 * g + 0] + __uint_as_float(bb.x << 16);
        v[1] = acc[i][j][4 * g + 1] + __uint_as_float(bb.x & 0xFFFF0000u);
        v[2] = acc[i][j][4 * g + 2] + __uint_as_float(bb.y << 16);
        v[3] = acc[i][j][4 * g + 3] + __uint_as_float(bb.y & 0xFFFF0000u);
        if (SILU) {
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = v[u] / (1.0f + __expf(-v[u]));
        }
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<uint2*>(orow + n) = o;
      }
    }
  }
}

namespace {

template <int TN, int TM, int WN, int WM, bool GATHER, bool SILU>
hipError_t launch_grouped_gemm(const bf16_t* A, const int32_t* row_token, const int32_t* offsets,
                               const bf16_t* W, const bf16_t* bias, bf16_t* out, int E, int N,
                               int K, int64_t rows_ub, hipStream_t st) {
  if (rows_ub <= 0) return hipSuccess;
  constexpr size_t lds = (size_t)2 * (TN + TM) * 8 * 16;
  auto kern = k_grouped_gemm<TN, TM, WN, WM, GATHER, SILU>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const int mt_ub = (int)((rows_ub + TM - 1) / TM) + E;
  const int n_tiles = (N + TN - 1) / TN;
  int64_t G = (int64_t)mt_ub * n_tiles;
  G = (G + 7) / 8 * 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)G), dim3(WN * WM * 64), lds, st, A, row_token, offsets,
                     W, bias, out, E, N, K, mt_ub, n_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_up_f32(const moe_shape& s, const void* x, const int32_t* row_token,
                             const int32_t* offsets, const void* w1, const void* b1, void* h,
                             hipStream_t st);
hipError_t launch_ffn_down_f32(const moe_shape& s, const void* h, const int32_t* offsets,
                               const void* w2, const void* b2, void* y, hipStream_t st);

hipError_t launch_ffn_up(const moe_shape& s, const void* x, const int32_t* row_token,
                         const int32_t* offsets, const void* w1, const void* b1, void* h,
                         hipStream_t st) {
  if (s.dtype != MOE_BF16) return launch_ffn_up_f32(s, x, row_token, offsets, w1, b1, h, st);
  return launch_grouped_gemm<256, 256, 2, 2, true, true>(
      (const bf16_t*)x, row_token, offsets, (const bf16_t*)w1, (const bf16_t*)b1, (bf16_t*)h,
      s.n_experts, s.d_ff, s.d_model, max_rows(s), st);
}

hipError_t launch_ffn_down(const moe_shape& s, const void* h, const int32_t* offsets,
                           const void* w2, const void* b2, void* y, hipStream_t st) {
  if (s.dtype != MOE_BF16) return launch_ffn_down_f32(s, h, offsets, w2, b2, y, st);
  return launch_grouped_gemm<256, 256, 2, 2, false, false>(
      (const bf16_t*)h, nullptr, offsets, (const bf16_t*)w2, (const bf16_t*)b2, (bf16_t*)y,
      s.n_experts, s.d_model, s.d_ff, max_rows(s), st);
}

}  // namespace moe
