// Expert FFN in bf16 on the matrix cores: two grouped GEMMs over the routed rows.
//
// Worked Example, trace of token 0: h = W1 x + b1, a = SiLU(h), y = W2 a + b2, each expert on
// its own batch of kept tokens; the closing paragraph of that page notes that the experts run
// side by side and the busiest one sets the wall-clock time.  Fused-MoE flow diagram (moe-vllm
// flow), boxes GEMM 1 and GEMM 2: the first GEMM reads its token rows through an index (the
// reorder happens on GEMM 1's read side) and each block works with one expert's weights.  Here
// the index is row_token[slot]; rows stay in expert-slot order until the combine.
//
//   GEMM 1 (GATHER, SILU): H[s, n] = SiLU(sum_k x[row_token[s], k] W1[e, n, k] + b1[e, n])
//   GEMM 2               : Y[s, n] = sum_k H[s, k] W2[e, n, k] + b2[e, n]
// for every kept slot s of expert e.  Both operands are K-contiguous ("NT" GEMM), the layout
// v_mfma_f32_32x32x16_bf16 wants: each lane feeds 8 consecutive K values of one row.
//
// Block tile: TN output features x TM slots, 4 waves of (TN/2) x (TM/2), each made of 32x32
// MFMA blocks with fp32 accumulators in AGPRs.  The weights are the MFMA "A" operand, the
// token rows the "B" operand.
//
// K pipeline: stages of 32 K; a ring of 4 stage buffers in LDS (32 KiB each for 256 x 256)
// filled by direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds) issued 3 stages ahead, so
// HBM / L2 latency is covered by three stages of MFMA work and the data never passes through
// VGPRs.  Each wave waits for its own loads of the next stage (vmcnt), then one barrier per
// stage publishes it; MFMA fragments are double-buffered in registers per 16-K step, so LDS
// reads of the next step overlap the MFMAs of the current one.  Row r of a stage buffer is
// 64 bytes (4 chunks of 16 B); chunk c is stored at c ^ ((r >> 2) & 3), which spreads the 16
// rows read by 16 consecutive lanes over all 64 LDS banks.  Loads go through buffer resources
// whose range covers only the tile's valid rows: out-of-range lanes (ragged rows, K tail)
// write zeros into LDS, so no branch guards a load.
//
// Epilogue: bias + activation + bf16 rounding per 16-accumulator group into an LDS tile, then
// coalesced 16-byte stores of whole output rows.
//
// Scheduling: the grid is an upper bound (the number of kept rows is only known on the
// device).  Workgroups are dealt round-robin over the 8 XCDs, so block b runs on XCD b % 8;
// blocks (b / 8) % 32 of round b / 256 on one XCD take one group of 8 token tiles x 4 weight
// tiles, so the 32 blocks sharing an L2 share both operands' streams.  Each block finds the
// expert of its token tile from expert_offsets with a wave prefix scan and exits if its tile
// does not exist.
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

constexpr int kGroupM = 8;               // token tiles per XCD group
constexpr int kGroupN = 32 / kGroupM;    // weight tiles per XCD group
constexpr uint32_t kOutOfRange = 0x80000000u;  // a byte offset beyond every buffer range used

// Buffer resource for raw (stride 0) loads of `bytes` bytes from `base`; reads past the range
// return zero.  Word 3 is the CDNA raw-buffer format.
__device__ __forceinline__ i32x4_t make_srd(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from the buffer at byte offset `voff` straight into LDS at
// lds_base + 16 * lane.  Written in assembly so the compiler does not order its own LDS reads
// behind these loads (it cannot tell which ring slot they fill); the kernel waits for them
// explicitly (vmcnt) before the barrier that publishes each stage, and waits for all of them
// before it exits.  The instruction has no destination registers.
__device__ __forceinline__ void lds_dma16(i32x4_t srd, uint32_t lds_base, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voff), "s"(srd)
      : "memory", "m0");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define MOE_WAIT_VMCNT_16() __builtin_amdgcn_s_waitcnt(0x4F70)
#define MOE_WAIT_VMCNT_8() __builtin_amdgcn_s_waitcnt(0x0F78)
#define MOE_WAIT_VMCNT_0() __builtin_amdgcn_s_waitcnt(0x0F70)

}  // namespace

template <int TN, int TM, bool GATHER, bool SILU>
__global__ __launch_bounds__(256, 1) void k_grouped_gemm(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ W,
    const bf16_t* __restrict__ bias, bf16_t* __restrict__ out, int E, int N, int K, int a_rows) {
  constexpr int WN = 2, WM = 2;              // waves along features / slots
  constexpr int kWaves = WN * WM;
  constexpr int kThreads = kWaves * 64;
  constexpr int BK = 32;                     // K per stage
  constexpr int NS = 4;                      // LDS ring depth (stages)
  constexpr int FN = TN / WN / 32;           // 32x32 blocks per wave along features
  constexpr int FM = TM / WM / 32;           // ... along slots
  constexpr int kRowsPerLoad = 16;           // one 1 KiB wave load = 16 rows x 64 B
  constexpr int kWLoads = TN / kRowsPerLoad / kWaves;  // weight loads per wave per stage
  constexpr int kXLoads = TM / kRowsPerLoad / kWaves;  // token-row loads per wave per stage
  constexpr int kStageBytes = (TN + TM) * BK * 2;
  static_assert(kWLoads + kXLoads == 8, "the vmcnt waits below assume 8 loads per stage");
  extern __shared__ uint4 smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int r32 = lane & 31, half = lane >> 5;

  // ---- token tiles per expert and their prefix (lane L owns experts 4L .. 4L+3)
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
  const int MT = __builtin_amdgcn_readfirstlane(__shfl(inc, 63, 64));
  const int NT = (N + TN - 1) / TN;
  const int NQ = (NT + kGroupN - 1) / kGroupN;
  const int NG = ((MT + kGroupM - 1) / kGroupM) * NQ;

  // ---- this block's tile
  const int xcd = blockIdx.x & 7, slot = (blockIdx.x >> 3) & 31, round = blockIdx.x >> 8;
  const int g = round * 8 + xcd;
  if (g >= NG) return;
  const int mt = (g / NQ) * kGroupM + slot % kGroupM;
  const int nt = (g % NQ) * kGroupN + slot / kGroupM;
  if (mt >= MT || nt >= NT) return;

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
  const int e = __builtin_amdgcn_readfirstlane(__shfl(esel, owner, 64) - 1);
  tstart = __builtin_amdgcn_readfirstlane(__shfl(tstart, owner, 64));
  const int row0 = offsets[e] + (mt - tstart) * TM;
  const int rows = min(TM, offsets[e + 1] - row0);
  const int n0 = nt * TN;
  const int wrows = min(TN, N - n0);

  // ---- load plan.  Lane i of a 1 KiB wave load fills row i/4 (of its 16), physical chunk i%4,
  // with logical chunk cch = (i%4) ^ ((row >> 2) & 3); (row >> 2) & 3 equals (i/16) & 3.
  const int lrow = lane >> 2;
  const int cch = (lane & 3) ^ ((lane >> 4) & 3);
  const i32x4_t wsrc = make_srd(W + ((int64_t)e * N + n0) * K, (uint32_t)(wrows * K * 2));
  i32x4_t xsrc;
  uint32_t xoff[kXLoads];
  if (GATHER) {
    xsrc = make_srd(A, (uint32_t)a_rows * (uint32_t)K * 2u);  // whole x (< 2 GiB, host-checked)
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int row = (wave * kXLoads + j) * kRowsPerLoad + lrow;
      xoff[j] = row < rows ? (uint32_t)(row_token[row0 + row] * K + cch * 8) * 2u : kOutOfRange;
    }
  } else {
    xsrc = make_srd(A + (int64_t)row0 * K, (uint32_t)(rows * K * 2));
#pragma unroll
    for (int j = 0; j < kXLoads; ++j)
      xoff[j] = (uint32_t)(((wave * kXLoads + j) * kRowsPerLoad + lrow) * K + cch * 8) * 2u;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;
  const int nk = (K + BK - 1) / BK;

#define MOE_ISSUE_STAGE(S)                                                                     \
  do {                                                                                         \
    const int k0_ = (S) * BK;                                                                  \
    const bool kin_ = k0_ + cch * 8 < K;                                                       \
    const uint32_t kb_ = (uint32_t)k0_ * 2u;                                                   \
    const uint32_t sb_ = lds0 + (uint32_t)(((S) % NS) * kStageBytes);                          \
    _Pragma("unroll") for (int j_ = 0; j_ < kWLoads; ++j_) {                                   \
      const int row_ = (wave * kWLoads + j_) * kRowsPerLoad + lrow;                            \
      lds_dma16(wsrc, sb_ + (uint32_t)((wave * kWLoads + j_) * kRowsPerLoad * 64),             \
                kin_ ? (uint32_t)((row_ * K + cch * 8) * 2) + kb_ : kOutOfRange);              \
    }                                                                                          \
    _Pragma("unroll") for (int j_ = 0; j_ < kXLoads; ++j_)                                     \
      lds_dma16(xsrc, sb_ + (uint32_t)(TN * 64 + (wave * kXLoads + j_) * kRowsPerLoad * 64),   \
                (kin_ && xoff[j_] != kOutOfRange) ? xoff[j_] + kb_ : kOutOfRange);             \
  } while (0)

#define MOE_READ_FRAGS(S, KK, F)                                                               \
  do {                                                                                         \
    const uint4* sb_ = smem + ((S) % NS) * (kStageBytes / 16);                                 \
    const int ch_ = (KK) * 2 + half;                                                           \
    _Pragma("unroll") for (int i_ = 0; i_ < FN; ++i_) {                                        \
      const int row_ = wn * (TN / WN) + i_ * 32 + r32;                                         \
      fa[F][i_] = as_bf16x8(sb_[row_ * 4 + (ch_ ^ ((row_ >> 2) & 3))]);                        \
    }                                                                                          \
    _Pragma("unroll") for (int j_ = 0; j_ < FM; ++j_) {                                        \
      const int row_ = wm * (TM / WM) + j_ * 32 + r32;                                         \
      fb[F][j_] = as_bf16x8(sb_[TN * 4 + row_ * 4 + (ch_ ^ ((row_ >> 2) & 3))]);               \
    }                                                                                          \
  } while (0)

#define MOE_MFMA_STEP(F)                                                                       \
  do {                                                                                         \
    _Pragma("unroll") for (int i_ = 0; i_ < FN; ++i_)                                          \
      _Pragma("unroll") for (int j_ = 0; j_ < FM; ++j_)                                        \
        acc[i_][j_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[F][i_], fb[F][j_],            \
                                                              acc[i_][j_], 0, 0, 0);           \
  } while (0)

  bf16x8_t fa[2][FN], fb[2][FM];
  f32x16_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // prologue: stages 0 .. NS-2 in flight; first 16-K step of stage 0 in registers
  MOE_ISSUE_STAGE(0);
  if (nk > 1) MOE_ISSUE_STAGE(1);
  if (nk > 2) MOE_ISSUE_STAGE(2);
  if (nk >= 3) MOE_WAIT_VMCNT_16();
  else if (nk == 2) MOE_WAIT_VMCNT_8();
  else MOE_WAIT_VMCNT_0();
  __syncthreads();
  MOE_READ_FRAGS(0, 0, 0);

  for (int kt = 0; kt < nk; ++kt) {
    // the slot of stage kt-1 is free: its last fragments were read before the last barrier
    if (kt + NS - 1 < nk) MOE_ISSUE_STAGE(kt + NS - 1);
    MOE_READ_FRAGS(kt, 1, 1);
    MOE_MFMA_STEP(0);
    // this wave's loads of stage kt+1 are done once at most the later stages' are pending
    const int pend = min(nk - 1, kt + NS - 1) - (kt + 1);
    if (pend >= 2) MOE_WAIT_VMCNT_16();
    else if (pend == 1) MOE_WAIT_VMCNT_8();
    else MOE_WAIT_VMCNT_0();
    __syncthreads();
    if (kt + 1 < nk) MOE_READ_FRAGS(kt + 1, 0, 0);
    MOE_MFMA_STEP(1);
  }
#undef MOE_ISSUE_STAGE
#undef MOE_READ_FRAGS
#undef MOE_MFMA_STEP

  // ---- epilogue.  Lane (r32, half) holds, for block (i, j), features
  // 32 i + 8 (v / 4) + 4 half + v % 4 of slot column 32 j + r32.  Bias + activation + bf16 go
  // into an LDS tile [TM slots][TN features] (row pitch TN * 2 + 16 bytes, so 16 consecutive
  // rows start on distinct banks); the tile then leaves as coalesced 16-byte stores.
  constexpr int kPitch = TN * 2 + 16;
  unsigned char* stile = reinterpret_cast<unsigned char*>(smem);
  __syncthreads();  // every wave is done reading the ring
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    uint2 bb[4];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int n = n0 + wn * (TN / WN) + i * 32 + 8 * g4 + 4 * half;
      bb[g4] = n < N ? *reinterpret_cast<const uint2*>(bias + (int64_t)e * N + n) : make_uint2(0, 0);
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      __builtin_amdgcn_sched_barrier(0);  // one block's 16 accumulators at a time
      const int tl = wm * (TM / WM) + j * 32 + r32;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int fl = wn * (TN / WN) + i * 32 + 8 * g4 + 4 * half;
        float v[4];
        v[0] = acc[i][j][4 * g4 + 0] + __uint_as_float(bb[g4].x << 16);
        v[1] = acc[i][j][4 * g4 + 1] + __uint_as_float(bb[g4].x & 0xFFFF0000u);
        v[2] = acc[i][j][4 * g4 + 2] + __uint_as_float(bb[g4].y << 16);
        v[3] = acc[i][j][4 * g4 + 3] + __uint_as_float(bb[g4].y & 0xFFFF0000u);
        if (SILU) {
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = v[u] * __builtin_amdgcn_rcpf(1.0f + __expf(-v[u]));
        }
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<uint2*>(stile + tl * kPitch + fl * 2) = o;
      }
    }
  }
  __syncthreads();
  constexpr int kChunksPerRow = TN / 8;
  const int ncols = min(TN, N - n0);
  for (int c = threadIdx.x; c < rows * kChunksPerRow; c += kThreads) {
    const int row = c / kChunksPerRow, ch = c % kChunksPerRow;
    if (ch * 8 < ncols)
      *reinterpret_cast<uint4*>(out + (int64_t)(row0 + row) * N + n0 + ch * 8) =
          *reinterpret_cast<const uint4*>(stile + row * kPitch + ch * 16);
  }
}

namespace {

template <int TN, int TM, bool GATHER, bool SILU>
hipError_t launch_grouped_gemm(const bf16_t* A, const int32_t* row_token, const int32_t* offsets,
                               const bf16_t* W, const bf16_t* bias, bf16_t* out, int E, int N,
                               int K, int a_rows, int64_t rows_ub, hipStream_t st) {
  if (rows_ub <= 0) return hipSuccess;
  constexpr size_t ring = (size_t)4 * (TN + TM) * 32 * 2;
  constexpr size_t tile = (size_t)TM * (TN * 2 + 16);
  constexpr size_t lds = ring > tile ? ring : tile;
  auto kern = k_grouped_gemm<TN, TM, GATHER, SILU>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  // upper bound on groups: token tiles <= rows_ub / TM + E
  const int64_t mt_ub = (rows_ub + TM - 1) / TM + E;
  const int64_t nt = (N + TN - 1) / TN;
  const int64_t nq = (nt + kGroupN - 1) / kGroupN;
  const int64_t ng_ub = (mt_ub + kGroupM - 1) / kGroupM * nq;
  const int64_t grid = (ng_ub + 7) / 8 * 256;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, st, A, row_token, offsets, W,
                     bias, out, E, N, K, a_rows);
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
  return launch_grouped_gemm<256, 256, true, true>(
      (const bf16_t*)x, row_token, offsets, (const bf16_t*)w1, (const bf16_t*)b1, (bf16_t*)h,
      s.n_experts, s.d_ff, s.d_model, (int)s.T, max_rows(s), st);
}

hipError_t launch_ffn_down(const moe_shape& s, const void* h, const int32_t* offsets,
                           const void* w2, const void* b2, void* y, hipStream_t st) {
  if (s.dtype != MOE_BF16) return launch_ffn_down_f32(s, h, offsets, w2, b2, y, st);
  return launch_grouped_gemm<256, 256, false, false>(
      (const bf16_t*)h, nullptr, offsets, (const bf16_t*)w2, (const bf16_t*)b2, (bf16_t*)y,
      s.n_experts, s.d_model, s.d_ff, (int)max_rows(s), max_rows(s), st);
}

}  // namespace moe
