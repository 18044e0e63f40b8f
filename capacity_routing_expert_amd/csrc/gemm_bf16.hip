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
// Block tile: TN output features x TM slots, 4 waves of (TN/2) x (TM/2) (or of (TN/4) x 32 for
// 32-slot tiles), each made of 32x32 MFMA blocks with fp32 accumulators in AGPRs.  The weights
// are the MFMA "A" operand, the token rows the "B" operand.  The large-batch up-projection runs
// 8 waves (2 x 4 of 128 x 64, two per SIMD) on its 256 x 256 tiles, so that one wave's MFMAs
// go on while the other waits on a load.  A second kernel (loader waves, below) runs the same
// stages with separate waves for the loads and for the MFMAs; it takes the large-batch
// down-projection.
//
// K pipeline: stages of BK = 32 K (64-byte rows) in a ring of NS = 4 stage buffers in LDS
// (32 KiB each for 256 x 256), filled by direct-to-LDS buffer loads (buffer_load_dwordx4 ...
// lds), so the data never passes through VGPRs.  Stage kt+NS is issued right after the barrier
// that ends the reads of stage kt, into the slot that barrier freed: each stage has three
// stages of MFMA work to arrive.  Its loads are spread one by one between the MFMAs of the
// following 16-K step, so a wave never waits on the load queue with an empty matrix pipe.  The
// loop body is the same on every step (stages past the last are issued as all-out-of-range
// loads that only write zeros), which keeps the vmcnt bookkeeping a constant.  MFMA fragments
// are double-buffered in registers per 16-K step, so LDS reads of the next step overlap the
// MFMAs of the current one.  Chunk c of row r of a stage buffer is stored at c ^ swz(r), which
// spreads the 16 rows read by 16 consecutive lanes over all 64 LDS banks.  Loads go through
// buffer resources whose range covers only the tile's valid rows: out-of-range lanes (ragged
// rows, K tail) write zeros into LDS, so no branch guards a load.  The kernel is templated on
// the tile, the stage depth (32 or 64) and the ring depth; 256 x 256 with 32-deep stages and a
// 4-deep ring measured fastest on the layer shapes here.
//
// Epilogue: bias + activation + bf16 rounding per 16-accumulator group into an LDS tile, then
// coalesced 16-byte stores of whole output rows.
//
// Timing: a launch can record its own kernel start and end in two events handed over with
// arm_launch_events (hipExtLaunchKernel), so nothing is queued between launches to time them.
//
// Scheduling: the grid is an upper bound (the number of kept rows is only known on the
// device).  Workgroups are dealt round-robin over the 8 XCDs, so block b runs on XCD b % 8;
// blocks (b / 8) % 32 of round b / 256 on one XCD take one group of token tiles x weight tiles
// (8 x 4, or 4 x 8 for the large up-projection), so the 32 blocks sharing an L2 share both
// operands' streams.  Each block finds the
// expert of its token tile from expert_offsets with a wave prefix scan and exits if its tile
// does not exist.
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// epilogue activation of a tile
constexpr int kActNone = 0;   // Y = acc + bias
constexpr int kActSilu = 1;   // H = SiLU(acc + bias)
constexpr int kActGated = 2;  // H = SiLU(gate) * up, gate and up rows of one weight tile, no bias

// Packed expert weights (MOE_WEIGHTS_PACKED): expert e's [rows, K] matrix is stored as
// [ceil(K / 32)][rows][32], so the 32-K slice of 256 consecutive rows that one stage of a large
// tile reads is one contiguous 16 KiB run (a row-major stage reads 256 runs of 64 bytes, 4-16
// KiB apart).  A 64-K stage of a decode tile reads two such blocks.
constexpr int kPackK = 32;

// where the rows of a tile go
constexpr int kOutSlots = 0;        // output row = slot (row0 + r)
constexpr int kOutPairs = 1;        // output row = out_row[slot] (dropless pair order)
constexpr int kOutPairsScaled = 2;  // ... and the row times row_scale[out_row[slot]]

// XCD groups of 32 blocks: GM token tiles x (32 / GM) weight tiles (template parameter of the
// kernels; 8 unless a launch says otherwise)
constexpr int kGroupBlocks = 32;
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
// before it exits.  The instruction has no destination registers.  M0 (the LDS address of the
// load) is written here and so named as clobbered; clang warns on every use that M0 is a
// reserved register, which is the point, so that warning is off for this function.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(i32x4_t srd, uint32_t lds_base, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voff), "s"(srd)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate that waits until at most n vector-memory loads are outstanding and leaves
// the other counters unconstrained (gfx9 encoding: vmcnt bits 3:0 and 15:14).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

}  // namespace

// Token tiles of height TM per expert, from expert_offsets (lane L owns experts 4L .. 4L+3):
// te[j] tiles of expert 4L+j, their exclusive prefix `excl` and inclusive `inc` over lanes,
// and the total MT (wave-uniform).
template <int TM>
struct TokenTiles {
  int te[4], excl, inc, MT;
  __device__ __forceinline__ TokenTiles(const int32_t* __restrict__ offsets, int E, int lane) {
    int local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ee = lane * 4 + j;
      const int kept = ee < E ? offsets[ee + 1] - offsets[ee] : 0;
      te[j] = (kept + TM - 1) / TM;
      local += te[j];
    }
    inc = local;
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(inc, off, 64);
      if (lane >= off) inc += o;
    }
    excl = inc - local;
    MT = __builtin_amdgcn_readfirstlane(__shfl(inc, 63, 64));
  }
  // expert and first row of token tile mt (wave-uniform)
  __device__ __forceinline__ void locate(const int32_t* __restrict__ offsets, int lane, int mt,
                                         int& e, int& row0, int& rows) const {
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
    e = __builtin_amdgcn_readfirstlane(__shfl(esel, owner, 64) - 1);
    tstart = __builtin_amdgcn_readfirstlane(__shfl(tstart, owner, 64));
    row0 = offsets[e] + (mt - tstart) * TM;
    rows = min(TM, offsets[e + 1] - row0);
  }
};

// Block -> (token tile, weight tile) of a grid of MT x NT tiles: block b runs on XCD b % 8, and
// the 32 blocks (b / 8) % 32 of round b / 256 on one XCD take one group of GM token tiles x
// 32 / GM weight tiles.  False if the block has no tile.
template <int GM>
__device__ __forceinline__ bool tile_of_block(int MT, int NT, int& mt, int& nt) {
  constexpr int GN = kGroupBlocks / GM;
  const int NQ = (NT + GN - 1) / GN;
  const int NG = ((MT + GM - 1) / GM) * NQ;
  const int xcd = blockIdx.x & 7, slot = (blockIdx.x >> 3) & 31, round = blockIdx.x >> 8;
  const int g = round * 8 + xcd;
  if (g >= NG) return false;
  mt = (g / NQ) * GM + slot % GM;
  nt = (g % NQ) * GN + slot / GM;
  return mt < MT && nt < NT;
}

// Blocks to launch for MT_ub x NT tiles in groups of GM x (32 / GM): whole rounds of 256.
template <int GM>
int64_t group_grid(int64_t mt_ub, int64_t nt) {
  constexpr int GN = kGroupBlocks / GM;
  const int64_t ng_ub = (mt_ub + GM - 1) / GM * ((nt + GN - 1) / GN);
  return (ng_ub + 7) / 8 * 256;
}

// One TN x TM output tile of expert e: token rows row0 .. row0 + rows - 1 (slots), features
// n0 .. n0 + TN - 1; NS-deep ring of BK-deep stages.
template <int TN, int TM, int BK, int NS, bool GATHER, int ACT, int OUT, bool WP, int NWV = 4,
          bool HP = false>
__device__ __forceinline__ void gemm_tile(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ row_token,
    const bf16_t* __restrict__ W, const bf16_t* __restrict__ bias, bf16_t* __restrict__ out,
    const int32_t* __restrict__ out_row, const float* __restrict__ row_scale, int N, int K,
    int a_rows, int e, int row0, int rows, int n0, int h_rows) {
  // waves along slots / features: 2 x 2; 4 x 2 for 8 waves (1 x 8 when the tile is at least
  // twice as wide as it is tall: every wave then holds 64 features x all the tile's slots); or
  // 1 x 4 for 32-slot tiles
  constexpr int WM = NWV == 8 ? (TN >= 2 * TM ? 1 : 4) : TM >= 64 ? 2 : 1, WN = NWV / WM;
  constexpr int kWaves = WN * WM;
  constexpr int kThreads = kWaves * 64;
  constexpr int KS = BK / 16;                // 16-K MFMA steps per stage
  constexpr int kChunks = BK / 8;            // 16-byte chunks per row of a stage
  constexpr int FN = TN / WN / 32;           // 32x32 blocks per wave along features
  constexpr int FM = TM / WM / 32;           // ... along slots
  constexpr int kRowsPerLoad = 64 / kChunks; // rows of one 1 KiB wave load
  constexpr int kWLoads = TN / kRowsPerLoad / kWaves;  // weight loads per wave per stage
  constexpr int kXLoads = TM / kRowsPerLoad / kWaves;  // token-row loads per wave per stage
  constexpr int kLoads = kWLoads + kXLoads;
  constexpr int kStageBytes = (TN + TM) * BK * 2;
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(FN >= 1 && FM >= 1 && kWLoads >= 1 && kXLoads >= 1, "tile too small");
  static_assert(TM % (kRowsPerLoad * kWaves) == 0 && TN % (kRowsPerLoad * kWaves) == 0,
                "whole wave loads per tile");
  static_assert(NS >= 2 && NS <= 8 && (NS - 1) * kLoads < 64, "ring depth (vmcnt holds 63)");
  constexpr bool GATED = ACT == kActGated;
  // output features per tile: a gated tile holds a gate row and an up row per output feature
  constexpr int TNO = GATED ? TN / 2 : TN;
  static_assert(!GATED || FN % 2 == 0, "gated tiles pair gate block i with up block i + FN/2");
  // Physical chunk of logical chunk c in row r is c ^ swz(r): the 16 rows read by 16
  // consecutive lanes then fall on distinct 16-byte bank groups (64 banks = 16 groups).
  auto swz = [](int r) { return BK == 32 ? (r >> 2) & 3 : (r >> 1) & 7; };
  extern __shared__ uint4 smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int r32 = lane & 31, half = lane >> 5;
  const int wrows = min(TN, N - n0);  // weight rows of the tile (non-gated)

  // ---- load plan.  A 1 KiB wave load fills kRowsPerLoad rows of kChunks 16-byte chunks: lane i
  // writes row i / kChunks, physical chunk p = i % kChunks, which holds logical chunk
  // p ^ swz(row) of that row.  The swizzle depends on the row's place in the stage buffer, so
  // the logical chunk of a lane can differ from one load of the stage to the next.
  const int lrow = lane / kChunks;
  const int pch = lane % kChunks;
  // Weight rows.  Non-gated: rows n0 .. n0 + TN - 1 of expert e's [N, K] block (rows past N
  // are out of the resource's range).  Gated: expert e's block is [2N, K], gate rows first;
  // LDS row rho of the feature portion wv = rho / P of wave column wv (P = TN / WN rows) holds
  // gate row n0 + wv P/2 + m (m = rho % P < P/2) or the up row N + n0 + wv P/2 + (m - P/2), so
  // gate block i and up block i + FN/2 of a wave cover the same output features; features past
  // N are out of range.
  static_assert(BK % kPackK == 0, "a stage reads whole packed blocks");
  const int NW = GATED ? 2 * N : N;                 // weight rows per expert
  const int KBW = (K + kPackK - 1) / kPackK;        // packed blocks per expert
  const i32x4_t wsrc =
      WP ? make_srd(W + (int64_t)e * KBW * NW * kPackK, (uint32_t)KBW * (uint32_t)NW * (kPackK * 2u))
      : GATED ? make_srd(W + (int64_t)e * 2 * N * K, (uint32_t)(2 * N * K * 2))
              : make_srd(W + ((int64_t)e * N + n0) * K, (uint32_t)(wrows * K * 2));
  // byte offset of K column kc of weight row r (expert-relative) in the packed layout
  auto packed_off = [&](int r, int kc) {
    return (uint32_t)(((kc / kPackK) * NW + r) * kPackK + kc % kPackK) * 2u;
  };
  uint32_t woff[kWLoads];  // byte offset of the lane's chunk at stage 0, or kOutOfRange
#pragma unroll
  for (int j = 0; j < kWLoads; ++j) {
    const int row = (wave * kWLoads + j) * kRowsPerLoad + lrow;
    const int c = pch ^ swz(row);
    if (GATED) {
      constexpr int P = TN / WN;  // weight rows of one wave column
      const int wv = row / P, m = row % P;
      const int feat = n0 + wv * (P / 2) + (m % (P / 2));
      const int grow = feat + (m >= P / 2 ? N : 0);
      woff[j] = feat < N && c * 8 < K ? (WP ? packed_off(grow, c * 8) : (uint32_t)(grow * K + c * 8) * 2u)
                                      : kOutOfRange;
    } else if (WP) {
      woff[j] = n0 + row < N && c * 8 < K ? packed_off(n0 + row, c * 8) : kOutOfRange;
    } else {
      woff[j] = c * 8 < K ? (uint32_t)(row * K + c * 8) * 2u : kOutOfRange;
    }
  }
  i32x4_t xsrc;
  uint32_t xoff[kXLoads];  // byte offset of the lane's chunk in stage 0, or kOutOfRange
  if (GATHER) {
    xsrc = make_srd(A, (uint32_t)a_rows * (uint32_t)K * 2u);  // whole x (< 2 GiB, host-checked)
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int row = (wave * kXLoads + j) * kRowsPerLoad + lrow;
      const int c = pch ^ swz(row);
      const int rt = row < rows ? row_token[row0 + row] : -1;  // -1: a zero row (padding)
      xoff[j] = rt >= 0 && c * 8 < K ? (uint32_t)(rt * K + c * 8) * 2u : kOutOfRange;
    }
  } else {
    xsrc = make_srd(A + (int64_t)row0 * K, (uint32_t)(rows * K * 2));
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int row = (wave * kXLoads + j) * kRowsPerLoad + lrow;
      const int c = pch ^ swz(row);
      xoff[j] = c * 8 < K ? (uint32_t)(row * K + c * 8) * 2u : kOutOfRange;
    }
  }
  // row scales of the slot columns this lane holds in the epilogue (fetched here, ahead of
  // the K loop, so the dependent index -> scale loads are long done when they are used)
  float rsc[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    rsc[j] = 1.0f;
    if (OUT == kOutPairsScaled) {
      const int tl = wm * (TM / WM) + j * 32 + r32;
      rsc[j] = tl < rows ? row_scale[out_row[row0 + tl]] : 0.0f;
    }
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;
  const int nk = (K + BK - 1) / BK;

// Load q of stage S (q < kWLoads: weight rows, else token rows), with k0_, kb_ and sb_ from
// MOE_STAGE_BASE.  A chunk at or past K (K tail, stages past the last) reads as zeros.
#define MOE_STAGE_BASE(S)                                                                      \
  const int k0_ = (S) * BK;                                                                    \
  const uint32_t kb_ = (uint32_t)k0_ * 2u;                                                     \
  const uint32_t kw_ = WP ? (uint32_t)(k0_ / kPackK) * (uint32_t)NW * (kPackK * 2u) : kb_;     \
  const uint32_t sb_ = lds0 + (uint32_t)(((S) % NS) * kStageBytes)
#define MOE_ISSUE_LOAD(q)                                                                      \
  do {                                                                                         \
    if ((q) < kWLoads) {                                                                       \
      const int g_ = wave * kWLoads + (q);                                                     \
      const int c_ = pch ^ swz(g_ * kRowsPerLoad + lrow);                                      \
      lds_dma16(wsrc, sb_ + (uint32_t)(g_ * 1024),                                             \
                (k0_ + c_ * 8 < K && woff[(q)] != kOutOfRange) ? woff[(q)] + kw_ : kOutOfRange); \
    } else {                                                                                   \
      const int j_ = (q) - kWLoads;                                                            \
      const int c_ = pch ^ swz((wave * kXLoads + j_) * kRowsPerLoad + lrow);                   \
      lds_dma16(xsrc, sb_ + (uint32_t)(TN * BK * 2 + (wave * kXLoads + j_) * 1024),            \
                (k0_ + c_ * 8 < K && xoff[j_] != kOutOfRange) ? xoff[j_] + kb_ : kOutOfRange); \
    }                                                                                          \
  } while (0)
#define MOE_ISSUE_STAGE(S)                                                                     \
  do {                                                                                         \
    MOE_STAGE_BASE(S);                                                                         \
    _Pragma("unroll") for (int q_ = 0; q_ < kLoads; ++q_) MOE_ISSUE_LOAD(q_);                  \
  } while (0)

#define MOE_READ_FRAGS(S, KK, F)                                                               \
  do {                                                                                         \
    const uint4* sb_ = smem + ((S) % NS) * (kStageBytes / 16);                                 \
    const int ch_ = (KK) * 2 + half;                                                           \
    _Pragma("unroll") for (int i_ = 0; i_ < FN; ++i_) {                                        \
      const int row_ = wn * (TN / WN) + i_ * 32 + r32;                                         \
      fa[F][i_] = as_bf16x8(sb_[row_ * kChunks + (ch_ ^ swz(row_))]);                          \
    }                                                                                          \
    _Pragma("unroll") for (int j_ = 0; j_ < FM; ++j_) {                                        \
      const int row_ = wm * (TM / WM) + j_ * 32 + r32;                                         \
      fb[F][j_] = as_bf16x8(sb_[TN * kChunks + row_ * kChunks + (ch_ ^ swz(row_))]);           \
    }                                                                                          \
  } while (0)

#define MOE_MFMA_STEP(F)                                                                       \
  do {                                                                                         \
    _Pragma("unroll") for (int i_ = 0; i_ < FN; ++i_)                                          \
      _Pragma("unroll") for (int j_ = 0; j_ < FM; ++j_)                                        \
        acc[i_][j_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[F][i_], fb[F][j_],            \
                                                              acc[i_][j_], 0, 0, 0);           \
  } while (0)

// Fragment q of 16-K step KK of stage S into register set F (q < FN: weight block q, else
// slot block q - FN).
#define MOE_READ_FRAG(S, KK, F, q)                                                             \
  do {                                                                                         \
    const uint4* sb_ = smem + ((S) % NS) * (kStageBytes / 16);                                 \
    const int ch_ = (KK) * 2 + half;                                                           \
    if ((q) < FN) {                                                                            \
      const int row_ = wn * (TN / WN) + (q) * 32 + r32;                                        \
      fa[F][(q)] = as_bf16x8(sb_[row_ * kChunks + (ch_ ^ swz(row_))]);                         \
    } else {                                                                                   \
      const int row_ = wm * (TM / WM) + ((q) - FN) * 32 + r32;                                 \
      fb[F][(q) - FN] = as_bf16x8(sb_[TN * kChunks + row_ * kChunks + (ch_ ^ swz(row_))]);     \
    }                                                                                          \
  } while (0)

// MFMA step F with the fragments of (S, KK) read into set G between the MFMAs, one after each
// of the first FN + FM MFMAs, and (LS >= 0) the loads of stage LS spread over the step as in
// MOE_MFMA_STEP_ISSUE.  Without the scheduling barriers the compiler issues all the reads
// ahead of the MFMAs, and the LDS then takes each wave's fragment reads in one burst.
#define MOE_MFMA_STEP_READ(F, S, KK, G, LS)                                                    \
  do {                                                                                         \
    MOE_STAGE_BASE((LS) < 0 ? 0 : (LS));                                                       \
    _Pragma("unroll") for (int m_ = 0; m_ < FN * FM; ++m_) {                                   \
      const int i_ = m_ / FM, j_ = m_ % FM;                                                    \
      acc[i_][j_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[F][i_], fb[F][j_], acc[i_][j_], \
                                                            0, 0, 0);                          \
      if (m_ < FN + FM) MOE_READ_FRAG(S, KK, G, m_);                                           \
      if ((LS) >= 0) {                                                                         \
        _Pragma("unroll") for (int q_ = 0; q_ < kLoads; ++q_)                                  \
          if (q_ * FN * FM / kLoads == m_) MOE_ISSUE_LOAD(q_);                                 \
      }                                                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                       \
    }                                                                                          \
  } while (0)

// MFMA step F with the loads of stage S spread between the MFMAs (load q after MFMA
// floor(q * FN * FM / kLoads)), so that the wave never stalls on the load queue while its
// matrix core has nothing queued.  The scheduling barriers keep this order.
#define MOE_MFMA_STEP_ISSUE(F, S)                                                              \
  do {                                                                                         \
    MOE_STAGE_BASE(S);                                                                         \
    _Pragma("unroll") for (int m_ = 0; m_ < FN * FM; ++m_) {                                   \
      const int i_ = m_ / FM, j_ = m_ % FM;                                                    \
      acc[i_][j_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[F][i_], fb[F][j_], acc[i_][j_], \
                                                            0, 0, 0);                          \
      _Pragma("unroll") for (int q_ = 0; q_ < kLoads; ++q_)                                    \
        if (q_ * FN * FM / kLoads == m_) MOE_ISSUE_LOAD(q_);                                   \
      __builtin_amdgcn_sched_barrier(0);                                                       \
    }                                                                                          \
  } while (0)

  bf16x8_t fa[2][FN], fb[2][FM];
  f32x16_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Ring: stage S lives in slot S % NS.  Stages 0 .. NS-1 are issued up front; stage kt+NS is
  // issued right after the barrier that ends the reads of stage kt, into the slot that barrier
  // freed, so a stage has NS-1 stages of MFMA work to arrive.  Stages past the last one are
  // issued too (every lane out of range: they write zeros into a slot no later stage reads),
  // which keeps the vmcnt bookkeeping the same on every step.
#pragma unroll
  for (int s0 = 0; s0 < NS; ++s0) MOE_ISSUE_STAGE(s0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * kLoads));
  __syncthreads();
  MOE_READ_FRAGS(0, 0, 0);

  // one fragment read between consecutive MFMAs needs at least as many MFMAs as reads per step
  constexpr bool kSpread = FN * FM >= FN + FM;
  static_assert(KS % 2 == 0, "the last step of a stage reads into set 0");
  for (int kt = 0; kt < nk; ++kt) {
    // 16-K steps 0 .. KS-2 of stage kt; fragments of the next step are read during each
#pragma unroll
    for (int kk = 0; kk < KS - 1; ++kk) {
      if constexpr (kSpread) {
        if (kk % 2 == 0)
          MOE_MFMA_STEP_READ(0, kt, kk + 1, 1, -1);
        else
          MOE_MFMA_STEP_READ(1, kt, kk + 1, 0, -1);
      } else if (kk % 2 == 0) {
        MOE_READ_FRAGS(kt, kk + 1, 1);
        MOE_MFMA_STEP(0);
      } else {
        MOE_READ_FRAGS(kt, kk + 1, 0);
        MOE_MFMA_STEP(1);
      }
    }
    // this wave's loads of stage kt+1 are done once only the NS-2 later stages are pending;
    // after the barrier every wave has read all of stage kt
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * kLoads));
    __syncthreads();
    // past the last stage the reads of stage kt+1 touch a slot nobody uses
    if constexpr (kSpread) {
      MOE_MFMA_STEP_READ(1, kt + 1, 0, 0, kt + NS);
    } else {
      MOE_READ_FRAGS(kt + 1, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      MOE_MFMA_STEP_ISSUE((KS - 1) % 2, kt + NS);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the zero-fill loads land before the LDS reuse
#undef MOE_STAGE_BASE
#undef MOE_ISSUE_LOAD
#undef MOE_ISSUE_STAGE
#undef MOE_READ_FRAGS
#undef MOE_MFMA_STEP
#undef MOE_MFMA_STEP_ISSUE
#undef MOE_READ_FRAG
#undef MOE_MFMA_STEP_READ

  // ---- epilogue.  Lane (r32, half) holds, for block (i, j), features
  // 32 i + 8 (v / 4) + 4 half + v % 4 of slot column 32 j + r32.  Bias + activation (+ row
  // scale) + bf16 go into an LDS tile [TM slots][TNO features] (row pitch TNO * 2 + 16 bytes,
  // so 16 consecutive rows start on distinct banks); the tile then leaves as coalesced 16-byte
  // stores, to rows row0 .. or, in pair order, to the rows out_row names (kept in LDS after the
  // tile).  A gated tile pairs gate block i with up block i + FN/2 (same lane layout, same
  // output features).
  constexpr int kPitch = TNO * 2 + 16;
  constexpr int FNO = GATED ? FN / 2 : FN;  // output blocks per wave along features
  unsigned char* stile = reinterpret_cast<unsigned char*>(smem);
  int32_t* srow = reinterpret_cast<int32_t*>(stile + TM * kPitch);
  __syncthreads();  // every wave is done reading the ring
  if (OUT != kOutSlots)
    for (int r = threadIdx.x; r < rows; r += kThreads) srow[r] = out_row[row0 + r];
#pragma unroll
  for (int i = 0; i < FNO; ++i) {
    uint2 bb[4];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int n = n0 + wn * (TNO / WN) + i * 32 + 8 * g4 + 4 * half;
      bb[g4] = !GATED && bias && n < N ? *reinterpret_cast<const uint2*>(bias + (int64_t)e * N + n)
                                       : make_uint2(0, 0);
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      __builtin_amdgcn_sched_barrier(0);  // one block's 16 accumulators at a time
      const int tl = wm * (TM / WM) + j * 32 + r32;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int fl = wn * (TNO / WN) + i * 32 + 8 * g4 + 4 * half;
        float v[4];
        if (GATED) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float gt = acc[i][j][4 * g4 + u], up = acc[i + FNO][j][4 * g4 + u];
            v[u] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
          }
        } else {
          v[0] = acc[i][j][4 * g4 + 0] + __uint_as_float(bb[g4].x << 16);
          v[1] = acc[i][j][4 * g4 + 1] + __uint_as_float(bb[g4].x & 0xFFFF0000u);
          v[2] = acc[i][j][4 * g4 + 2] + __uint_as_float(bb[g4].y << 16);
          v[3] = acc[i][j][4 * g4 + 3] + __uint_as_float(bb[g4].y & 0xFFFF0000u);
          if (ACT == kActSilu) {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = v[u] * __builtin_amdgcn_rcpf(1.0f + __expf(-v[u]));
          }
        }
        if (OUT == kOutPairsScaled) {
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] *= rsc[j];
        }
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(stile + tl * kPitch + fl * 2) = o;
      }
    }
  }
  __syncthreads();
  constexpr int kChunksPerRow = TNO / 8;
  const int ncols = min(TNO, N - n0);
  if constexpr (HP) {
    // H in 32-column blocks (slot order, N a multiple of 32): element (slot r, feature n) at
    // ((n / 32) h_rows + r) 32 + n % 32.  Thread c writes chunk c % 4 of row (c / 4) % rows of
    // the tile's 32-column block c / (4 rows), so consecutive threads fill consecutive 16 bytes.
    static_assert(OUT == kOutSlots && TNO % 32 == 0, "packed H holds slot-order rows");
    for (int c = threadIdx.x; c < rows * kChunksPerRow; c += kThreads) {
      const int q = c & 3, rb = c >> 2;
      const int row = rb % rows, blk = rb / rows;
      const int n = n0 + blk * 32 + q * 8;
      if (n < N)
        *reinterpret_cast<uint4*>(out + ((int64_t)(n >> 5) * h_rows + row0 + row) * 32 + q * 8) =
            *reinterpret_cast<const uint4*>(stile + row * kPitch + (blk * 32 + q * 8) * 2);
    }
    return;
  }
  for (int c = threadIdx.x; c < rows * kChunksPerRow; c += kThreads) {
    const int row = c / kChunksPerRow, ch = c % kChunksPerRow;
    const int64_t orow = OUT != kOutSlots ? (int64_t)srow[row] : (int64_t)(row0 + row);
    if (ch * 8 < ncols)
      *reinterpret_cast<uint4*>(out + orow * N + n0 + ch * 8) =
          *reinterpret_cast<const uint4*>(stile + row * kPitch + ch * 16);
  }
}

// The grouped GEMM kernel.  Each block works out the token tiles of every expert from
// expert_offsets (device memory: the kept-row counts are only known on the device), finds its
// own (expert, token tile, feature tile) and exits if that tile does not exist.
template <int TN, int TM, int BK, int NS, int MINB, bool GATHER, int ACT, int OUT, bool WP,
          int NWV = 4, int GM = 8, bool HP = false>
__global__ __launch_bounds__(64 * NWV, MINB) void k_grouped_gemm(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ W,
    const bf16_t* __restrict__ bias, bf16_t* __restrict__ out, const int32_t* __restrict__ out_row,
    const float* __restrict__ row_scale, int E, int N, int K, int a_rows, int h_rows) {
  const int lane = threadIdx.x & 63;
  constexpr int TNO = ACT == kActGated ? TN / 2 : TN;  // output features per tile
  const int NT = (N + TNO - 1) / TNO;
  const TokenTiles<TM> tt(offsets, E, lane);
  int mt, nt, e, row0, rows;
  if (!tile_of_block<GM>(tt.MT, NT, mt, nt)) return;
  tt.locate(offsets, lane, mt, e, row0, rows);
  gemm_tile<TN, TM, BK, NS, GATHER, ACT, OUT, WP, NWV, HP>(
      A, row_token, W, bias, out, out_row, row_scale, N, K, a_rows, e, row0, rows, nt * TNO,
      h_rows);
}

// ---------------------------------------------------------------- loader waves
// The large-batch down-projection (GEMM 2: no activation) runs on 512-thread blocks of 256 x 192
// tiles.  Waves 4-7 only issue the direct-to-LDS loads of the NS-deep ring of 32-K stages;
// waves 0-3 only read LDS fragments and run the MFMAs (128 features x 96 slots each, fp32
// accumulators in VGPRs, two waves per SIMD).  The load issue, which can stall a wave behind a
// busy memory pipeline, then no longer holds up the matrix cores.  One barrier per stage: the
// loader waves pass it once this wave's loads of stage kt+1 have landed, the MFMA waves once
// they have read all of stage kt, and right after it the loaders refill the freed slot with
// stage kt+NS.  The stage layout, swizzle, MFMA blocks and K order are those of gemm_tile, so
// every output element sums the same products in the same order (bit-identical results).
template <int TN, int TM, int NS, bool GATHER, int ACT, int OUT, bool WP, bool AP = false>
__device__ __forceinline__ void gemm_tile_loaders(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ row_token,
    const bf16_t* __restrict__ W, const bf16_t* __restrict__ bias, bf16_t* __restrict__ out,
    const int32_t* __restrict__ out_row, const float* __restrict__ row_scale, int N, int K,
    int a_rows, int e, int row0, int rows, int n0) {
  constexpr int BK = 32, WN = 2, WM = 2, kChunks = 4, kRowsPerLoad = 16;
  constexpr int FN = TN / WN / 32, FM = TM / WM / 32;
  constexpr int kLoaders = 4, kThreads = 512;
  constexpr int kWLoads = TN / kRowsPerLoad / kLoaders;  // per loader wave and stage
  constexpr int kXLoads = TM / kRowsPerLoad / kLoaders;
  constexpr int kLoads = kWLoads + kXLoads;
  constexpr int kStageBytes = (TN + TM) * BK * 2;
  static_assert(TN % (kRowsPerLoad * kLoaders) == 0 && TM % (kRowsPerLoad * kLoaders) == 0 &&
                    FN >= 1 && FM >= 1 && NS >= 2 && (NS - 1) * kLoads < 64,
                "tile shape");
  static_assert(BK % kPackK == 0, "a stage reads whole packed blocks");
  static_assert(ACT == kActNone, "loader waves run the down-projection (no activation)");
  auto swz = [](int r) { return (r >> 2) & 3; };
  extern __shared__ uint4 smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;
  const int nk = (K + BK - 1) / BK;
  const int wrows = min(TN, N - n0);
  constexpr int kPitch = TN * 2 + 16;  // epilogue staging tile [TM][TN] bf16, padded rows
  unsigned char* stile = reinterpret_cast<unsigned char*>(smem);
  int32_t* srow = reinterpret_cast<int32_t*>(stile + TM * kPitch);

  if (wave >= 4) {
    // ---- loader waves: the load plan of gemm_tile, split over 4 waves instead of 4 MFMA waves
    const int lw = wave - 4;
    const int lrow = lane / kChunks, pch = lane % kChunks;
    const int KBW = (K + kPackK - 1) / kPackK;
    const i32x4_t wsrc =
        WP ? make_srd(W + (int64_t)e * KBW * N * kPackK, (uint32_t)KBW * (uint32_t)N * (kPackK * 2u))
           : make_srd(W + ((int64_t)e * N + n0) * K, (uint32_t)(wrows * K * 2));
    uint32_t woff[kWLoads];
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) {
      const int row = (lw * kWLoads + j) * kRowsPerLoad + lrow;
      const int c = pch ^ swz(row);
      if (WP)
        woff[j] = n0 + row < N && c * 8 < K
                      ? (uint32_t)(((c * 8 / kPackK) * N + n0 + row) * kPackK + (c * 8) % kPackK) * 2u
                      : kOutOfRange;
      else
        woff[j] = c * 8 < K ? (uint32_t)(row * K + c * 8) * 2u : kOutOfRange;
    }
    i32x4_t xsrc;
    uint32_t xoff[kXLoads];
    if (GATHER) {
      xsrc = make_srd(A, (uint32_t)a_rows * (uint32_t)K * 2u);
#pragma unroll
      for (int j = 0; j < kXLoads; ++j) {
        const int row = (lw * kXLoads + j) * kRowsPerLoad + lrow;
        const int c = pch ^ swz(row);
        const int rt = row < rows ? row_token[row0 + row] : -1;  // -1: a zero row (padding)
        xoff[j] = rt >= 0 && c * 8 < K ? (uint32_t)(rt * K + c * 8) * 2u : kOutOfRange;
      }
    } else if (AP) {
      // A in 32-column blocks of a_rows rows (written so by the up-projection): each 32-K
      // stage of the tile's rows is one contiguous run, row r's piece at (r * 32 + c * 8) * 2
      // bytes past block k0 / 32 (a_rows * 64 bytes each)
      xsrc = make_srd(A, (uint32_t)a_rows * (uint32_t)K * 2u);
#pragma unroll
      for (int j = 0; j < kXLoads; ++j) {
        const int row = (lw * kXLoads + j) * kRowsPerLoad + lrow;
        const int c = pch ^ swz(row);
        xoff[j] = row < rows ? (uint32_t)((row0 + row) * 32 + c * 8) * 2u : kOutOfRange;
      }
    } else {
      xsrc = make_srd(A + (int64_t)row0 * K, (uint32_t)(rows * K * 2));
#pragma unroll
      for (int j = 0; j < kXLoads; ++j) {
        const int row = (lw * kXLoads + j) * kRowsPerLoad + lrow;
        const int c = pch ^ swz(row);
        xoff[j] = c * 8 < K ? (uint32_t)(row * K + c * 8) * 2u : kOutOfRange;
      }
    }
    static_assert(!AP || !GATHER, "packed A rows are read in slot order");
    // stage S into slot S % NS; chunks at or past K (K tail, stages past the last) read as zeros
    auto issue = [&](int S) {
      const int k0 = S * BK;
      const uint32_t kb = (uint32_t)k0 * 2u;
      const uint32_t kw = WP ? (uint32_t)(k0 / kPackK) * (uint32_t)N * (kPackK * 2u) : kb;
      const uint32_t ka = AP ? (uint32_t)(k0 / kPackK) * (uint32_t)a_rows * (kPackK * 2u) : kb;
      const uint32_t sb = lds0 + (uint32_t)((S % NS) * kStageBytes);
#pragma unroll
      for (int j = 0; j < kWLoads; ++j) {
        const int g = lw * kWLoads + j;
        const int c = pch ^ swz(g * kRowsPerLoad + lrow);
        lds_dma16(wsrc, sb + (uint32_t)(g * 1024),
                  (k0 + c * 8 < K && woff[j] != kOutOfRange) ? woff[j] + kw : kOutOfRange);
      }
#pragma unroll
      for (int j = 0; j < kXLoads; ++j) {
        const int g = lw * kXLoads + j;
        const int c = pch ^ swz(g * kRowsPerLoad + lrow);
        lds_dma16(xsrc, sb + (uint32_t)(TN * BK * 2 + g * 1024),
                  (k0 + c * 8 < K && xoff[j] != kOutOfRange) ? xoff[j] + ka : kOutOfRange);
      }
    };
    for (int s0 = 0; s0 < NS; ++s0) issue(s0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * kLoads));
    __syncthreads();  // stage 0 is in
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * kLoads));  // this wave's stage kt+1
      __syncthreads();  // stage kt+1 is in, stage kt is read
      issue(kt + NS);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the zero-fill loads land before the LDS reuse
    __syncthreads();                           // the ring is free for the staging tile
    if (OUT != kOutSlots)
      for (int r = threadIdx.x - 256; r < rows; r += 256) srow[r] = out_row[row0 + r];
  } else {
    // ---- MFMA waves
    const int wn = wave % WN, wm = wave / WN;
    const int r32 = lane & 31, half = lane >> 5;
    float rsc[FM];  // row scales of this lane's slot columns, fetched ahead of the K loop
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      rsc[j] = 1.0f;
      if (OUT == kOutPairsScaled) {
        const int tl = wm * (TM / WM) + j * 32 + r32;
        rsc[j] = tl < rows ? row_scale[out_row[row0 + tl]] : 0.0f;
      }
    }
    bf16x8_t fa[2][FN], fb[2][FM];
    f32x16_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    // fragments of 16-K step kk of stage S into register set F
    // fragment q (q < FN: weight block q, else slot block q - FN) of 16-K step kk of stage S
    // into register set F
    auto read1 = [&](int S, int kk, int F, int q) {
      const uint4* sb = smem + (S % NS) * (kStageBytes / 16);
      const int ch = kk * 2 + half;
      if (q < FN) {
        const int row = wn * (TN / WN) + q * 32 + r32;
        fa[F][q] = as_bf16x8(sb[row * kChunks + (ch ^ swz(row))]);
      } else {
        const int row = wm * (TM / WM) + (q - FN) * 32 + r32;
        fb[F][q - FN] = as_bf16x8(sb[TN * kChunks + row * kChunks + (ch ^ swz(row))]);
      }
    };
    // the MFMAs of register set F, with the fragments of (S, kk) read into set G between them,
    // one after each of the first FN + FM MFMAs.  The scheduling barriers keep that order: the
    // compiler otherwise issues all the reads ahead of the MFMAs, and the LDS then sees the
    // fragment reads in bursts (lab, same bits: down-projection mid 171 -> 154 us, collapse
    // 4.97 -> 4.44 ms, 64-expert fine 248 -> 236 us).  The gathering form (pair order) keeps
    // the reads ahead of the MFMAs: interleaved, its extra row registers spill.
    auto mfma_read = [&](int F, int S, int kk, int G) {
      if constexpr (GATHER) {
#pragma unroll
        for (int q = 0; q < FN + FM; ++q) read1(S, kk, G, q);
#pragma unroll
        for (int m = 0; m < FN * FM; ++m)
          acc[m / FM][m % FM] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              fa[F][m / FM], fb[F][m % FM], acc[m / FM][m % FM], 0, 0, 0);
      } else {
#pragma unroll
        for (int m = 0; m < FN * FM; ++m) {
          const int i = m / FM, j = m % FM;
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[F][i], fb[F][j], acc[i][j], 0, 0, 0);
          if (m < FN + FM) read1(S, kk, G, m);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    static_assert(FN * FM >= FN + FM, "one fragment read per MFMA at most");
    __syncthreads();  // stage 0 is in
#pragma unroll
    for (int q = 0; q < FN + FM; ++q) read1(0, 0, 0, q);
    for (int kt = 0; kt < nk; ++kt) {
      mfma_read(0, kt, 1, 1);
      __syncthreads();  // stage kt+1 is in, stage kt is read
      mfma_read(1, kt + 1, 0, 0);  // past the last stage this reads a slot nobody uses
    }
    __syncthreads();  // the ring is free for the staging tile
    // bias (+ row scale) + bf16 into the staging tile: lane (r32, half) holds, for block (i, j),
    // features 32 i + 8 (v / 4) + 4 half + v % 4 of slot column 32 j + r32
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      uint2 bb[4];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int n = n0 + wn * (TN / WN) + i * 32 + 8 * g4 + 4 * half;
        bb[g4] = bias && n < N ? *reinterpret_cast<const uint2*>(bias + (int64_t)e * N + n)
                               : make_uint2(0, 0);
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
          if (OUT == kOutPairsScaled) {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] *= rsc[j];
          }
          uint2 o;
          o.x = pack_bf16x2(v[0], v[1]);
          o.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(stile + tl * kPitch + fl * 2) = o;
        }
      }
    }
  }
  __syncthreads();  // staging tile and output rows complete
  // coalesced 16-byte stores of whole output rows by all 512 threads
  constexpr int kChunksPerRow = TN / 8;
  const int ncols = min(TN, N - n0);
  for (int c = threadIdx.x; c < rows * kChunksPerRow; c += kThreads) {
    const int row = c / kChunksPerRow, ch = c % kChunksPerRow;
    const int64_t orow = OUT != kOutSlots ? (int64_t)srow[row] : (int64_t)(row0 + row);
    if (ch * 8 < ncols)
      *reinterpret_cast<uint4*>(out + orow * N + n0 + ch * 8) =
          *reinterpret_cast<const uint4*>(stile + row * kPitch + ch * 16);
  }
}

template <int TN, int TM, int NS, bool GATHER, int ACT, int OUT, bool WP, bool AP = false>
__global__ __launch_bounds__(512, 1) void k_grouped_gemm_loaders(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ W,
    const bf16_t* __restrict__ bias, bf16_t* __restrict__ out, const int32_t* __restrict__ out_row,
    const float* __restrict__ row_scale, int E, int N, int K, int a_rows) {
  const int lane = threadIdx.x & 63;
  const int NT = (N + TN - 1) / TN;
  const TokenTiles<TM> tt(offsets, E, lane);
  int mt, nt, e, row0, rows;
  if (!tile_of_block<8>(tt.MT, NT, mt, nt)) return;  // block-uniform
  tt.locate(offsets, lane, mt, e, row0, rows);
  gemm_tile_loaders<TN, TM, NS, GATHER, ACT, OUT, WP, AP>(A, row_token, W, bias, out, out_row,
                                                     row_scale, N, K, a_rows, e, row0, rows,
                                                     nt * TN);
}

// ---------------------------------------------------------------- weight packing
// [E, rows, cols] row-major -> [E, ceil(cols / 32), rows, 32], K columns past cols zero.  One
// thread per 16-byte chunk of the packed array (cols is a multiple of 8 in bf16).
__global__ __launch_bounds__(256) void k_pack_weights(const bf16_t* __restrict__ w,
                                                      bf16_t* __restrict__ wp, int64_t E, int rows,
                                                      int cols) {
  const int kb_n = (cols + kPackK - 1) / kPackK;
  const int64_t chunks = E * kb_n * (int64_t)rows * (kPackK / 8);
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * 256) {
    const int q = (int)(c % (kPackK / 8));
    const int64_t r_all = c / (kPackK / 8);  // (e, kb, row)
    const int row = (int)(r_all % rows);
    const int64_t ekb = r_all / rows;
    const int kb = (int)(ekb % kb_n);
    const int64_t e = ekb / kb_n;
    const int col = kb * kPackK + q * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (col < cols) v = *reinterpret_cast<const uint4*>(w + (e * rows + row) * (int64_t)cols + col);
    *reinterpret_cast<uint4*>(wp + c * 8) = v;
  }
}

int64_t packed_weight_elems(int64_t E, int rows, int cols) {
  return E * ((cols + kPackK - 1) / kPackK) * (int64_t)rows * kPackK;
}

hipError_t launch_pack_weights(const void* w, void* wp, int64_t E, int rows, int cols,
                               hipStream_t st) {
  const int64_t chunks = packed_weight_elems(E, rows, cols) / 8;
  if (chunks <= 0) return hipSuccess;
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(k_pack_weights, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256),
                     0, st, (const bf16_t*)w, (bf16_t*)wp, E, rows, cols);
  return hipGetLastError();
}

namespace {
thread_local hipEvent_t g_gemm_start = nullptr, g_gemm_stop = nullptr;
}  // namespace

void arm_launch_events(hipEvent_t start, hipEvent_t stop) {
  g_gemm_start = start;
  g_gemm_stop = stop;
}

bool take_launch_events(hipEvent_t* start, hipEvent_t* stop) {
  if (!g_gemm_start && !g_gemm_stop) return false;
  *start = g_gemm_start;
  *stop = g_gemm_stop;
  g_gemm_start = g_gemm_stop = nullptr;
  return true;
}

namespace {

constexpr size_t tile_lds(int TN, int TM, int BK, int NS, bool out_rows) {
  const size_t ring = (size_t)NS * (TN + TM) * BK * 2;      // stage ring
  const size_t tile = (size_t)TM * (TN * 2 + 16)            // epilogue staging tile
                      + (out_rows ? (size_t)TM * 4 : 0);    // + the output row of each slot
  return ring > tile ? ring : tile;
}

template <int TN, int TM, int BK, int NS, int MINB, bool GATHER, int ACT, int OUT, bool WP,
          int NWV = 4, int GM = 8, bool HP = false>
hipError_t launch_grouped_gemm(const bf16_t* A, const int32_t* row_token, const int32_t* offsets,
                               const bf16_t* W, const bf16_t* bias, bf16_t* out, int E, int N,
                               int K, int a_rows, int64_t rows_ub, hipStream_t st,
                               const int32_t* out_row = nullptr,
                               const float* row_scale = nullptr) {
  if (rows_ub <= 0) return hipSuccess;
  constexpr size_t lds = tile_lds(TN, TM, BK, NS, OUT != kOutSlots);
  static_assert(lds * MINB <= 160 * 1024, "LDS per compute unit");
  auto kern = k_grouped_gemm<TN, TM, BK, NS, MINB, GATHER, ACT, OUT, WP, NWV, GM, HP>;
  static std::atomic<bool> lds_allowed[kMaxDevices];
  if (hipError_t err = allow_dynamic_lds((const void*)kern, (int)lds, lds_allowed);
      err != hipSuccess)
    return err;
  // upper bound on groups: token tiles <= rows_ub / TM + E
  const int64_t mt_ub = (rows_ub + TM - 1) / TM + E;
  constexpr int TNO = ACT == kActGated ? TN / 2 : TN;
  const int64_t grid = group_grid<GM>(mt_ub, (N + TNO - 1) / TNO);
  const int h_rows = HP ? (int)rows_ub : 0;  // packed H: the rows of the output array
  hipEvent_t t0, t1;
  if (take_launch_events(&t0, &t1))
    hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * NWV), lds, st, t0, t1, 0, A,
                          row_token, offsets, W, bias, out, out_row, row_scale, E, N, K, a_rows,
                          h_rows);
  else
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * NWV), lds, st, A, row_token, offsets, W,
                       bias, out, out_row, row_scale, E, N, K, a_rows, h_rows);
  return hipGetLastError();
}

template <int TN, int TM, int NS, bool GATHER, int ACT, int OUT, bool WP, bool AP = false>
hipError_t launch_grouped_gemm_loaders(const bf16_t* A, const int32_t* row_token,
                                       const int32_t* offsets, const bf16_t* W, const bf16_t* bias,
                                       bf16_t* out, int E, int N, int K, int a_rows,
                                       int64_t rows_ub, hipStream_t st,
                                       const int32_t* out_row = nullptr,
                                       const float* row_scale = nullptr) {
  if (rows_ub <= 0) return hipSuccess;
  constexpr size_t ring = (size_t)NS * (TN + TM) * 32 * 2;
  constexpr size_t tile = (size_t)TM * (TN * 2 + 16) + (OUT != kOutSlots ? (size_t)TM * 4 : 0);
  constexpr size_t lds = ring > tile ? ring : tile;
  static_assert(lds <= 160 * 1024, "LDS per compute unit");
  auto kern = k_grouped_gemm_loaders<TN, TM, NS, GATHER, ACT, OUT, WP, AP>;
  static std::atomic<bool> lds_allowed[kMaxDevices];
  if (hipError_t err = allow_dynamic_lds((const void*)kern, (int)lds, lds_allowed);
      err != hipSuccess)
    return err;
  const int64_t mt_ub = (rows_ub + TM - 1) / TM + E;  // token tiles <= rows_ub / TM + E
  const int64_t grid = group_grid<8>(mt_ub, (N + TN - 1) / TN);
  hipEvent_t t0, t1;
  if (take_launch_events(&t0, &t1))
    hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, st, t0, t1, 0, A,
                          row_token, offsets, W, bias, out, out_row, row_scale, E, N, K, a_rows);
  else
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, st, A, row_token, offsets, W,
                       bias, out, out_row, row_scale, E, N, K, a_rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_up_f32(const moe_shape& s, const void* x, const int32_t* row_token,
                             const int32_t* offsets, const void* w1, const void* b1, void* h,
                             int64_t rows_ub, hipStream_t st);
hipError_t launch_ffn_down_f32(const moe_shape& s, const void* h, const int32_t* offsets,
                               const void* w2, const void* b2, void* y, int64_t rows_ub,
                               hipStream_t st);

// Few rows per expert (decode-sized batches): the layer is bound by streaming the expert
// weights, and 256 x 256 tiles would leave most compute units idle (8 experts x d_model / 256
// tiles for the down-projection).  Small tiles with 64-deep stages and two blocks per compute
// unit put every unit to work on its own weight rows: 64 x 64 for the down-projection, 128 x 32
// (128 weight rows, 32 slots) for the up-projection, whose d_ff / 128 feature tiles per expert
// still fill the GPU.  An expert with more than 32 kept rows then takes several token tiles,
// which stream its weight rows again (mostly from L2: the tiles of one weight tile run side by
// side on one XCD).
static bool skinny(const moe_shape& s, int64_t rows_ub) {
  return rows_ub <= (int64_t)64 * s.n_experts;
}

// H (GEMM 1's output, GEMM 2's input, slot order) is stored in 32-column blocks, [d_ff / 32,
// rows, 32], whenever the large tiles run: the down-projection's loader waves then read each
// 32-K stage of a token tile as one contiguous 16 KiB run instead of 64-byte pieces of rows
// d_ff * 2 bytes apart (same bits; stage times in the layer: GEMM 2 mid 180 -> 161 us, 64-expert
// fine 271 -> 235 us, collapse 5.23 -> 4.73 ms, GEMM 1 unchanged by its block-ordered stores).
// Needs d_ff a multiple of 32 and H within a buffer resource's 32-bit range; the
// two GEMMs of a call see the same shape and row bound, so they agree on the layout.
static bool h_packed(const moe_shape& s, int64_t rows_ub) {
  return s.dtype == MOE_BF16 && !skinny(s, rows_ub) && s.d_ff % 32 == 0 &&
         rows_ub * (int64_t)s.d_ff * 2 < ((int64_t)1 << 31);
}

namespace {

// The tile configurations: large batches, and decode-sized ones (skinny); the gated expert's
// tiles hold a gate row and an up row per output feature.
template <int ACT, int OUT, bool GATHER, bool WP, bool HP = false>
hipError_t run_gemm(bool small, const bf16_t* A, const int32_t* row_token, const int32_t* offsets,
                    const bf16_t* W, const bf16_t* bias, bf16_t* out, int E, int N, int K,
                    int a_rows, int64_t rows_ub, hipStream_t st, const int32_t* out_row,
                    const float* row_scale) {
  if constexpr (ACT == kActGated) {
    if (small)
      return launch_grouped_gemm<128, 64, 64, 3, 2, GATHER, ACT, OUT, WP>(
          A, row_token, offsets, W, bias, out, E, N, K, a_rows, rows_ub, st, out_row, row_scale);
  } else if constexpr (ACT == kActSilu) {
    // the up-projection's many feature tiles: 128 weight rows x 32 slots, so a block streams
    // twice the weight rows per stage and the grid is half as many blocks
    if (small)
      return launch_grouped_gemm<128, 32, 64, 3, 2, GATHER, ACT, OUT, WP>(
          A, row_token, offsets, W, bias, out, E, N, K, a_rows, rows_ub, st, out_row, row_scale);
  } else {
    if (small)
      return launch_grouped_gemm<64, 64, 64, 4, 2, GATHER, ACT, OUT, WP>(
          A, row_token, offsets, W, bias, out, E, N, K, a_rows, rows_ub, st, out_row, row_scale);
  }
  // Large batches.  The down-projection runs on loader waves (256 x 192 tiles); the
  // up-projection on 8-wave blocks of 256 x 256 tiles, two waves of 128 x 64 per SIMD, so one
  // wave's MFMAs run while the other waits on a load (mid layer GEMM 1: 215 -> 195 us).  The
  // up-projection's XCD groups are 4 token tiles x 8 weight tiles: a token tile's 8 weight tiles
  // then share its gathered rows in one L2 (64-expert fine layer GEMM 1: 395 -> 350 us, collapse
  // 5.20 -> 5.01 ms, mid unchanged; the down-projection keeps 8 x 4).
  // With 32 experts or more (many experts with few rows), the up-projection takes tiles of 512
  // features x 128 slots instead: half the token tile, so less padding in each expert's last
  // tile (lab, same bits: 64-expert fine layer 357 -> 311 us; mid 240 -> 246 us and collapse
  // 5.16 -> 5.80 ms, so only there).
  // HP: H in 32-column blocks (written by the up-projection, read by the down-projection)
  if constexpr (ACT == kActNone) {
    return launch_grouped_gemm_loaders<256, 192, 4, GATHER, ACT, OUT, WP, HP && !GATHER>(
        A, row_token, offsets, W, bias, out, E, N, K, a_rows, rows_ub, st, out_row, row_scale);
  } else {
    if (E >= 32)
      return launch_grouped_gemm<512, 128, 32, 4, 1, GATHER, ACT, OUT, WP, 8, 4, HP>(
          A, row_token, offsets, W, bias, out, E, N, K, a_rows, rows_ub, st, out_row, row_scale);
    return launch_grouped_gemm<256, 256, 32, 4, 1, GATHER, ACT, OUT, WP, 8, 4, HP>(
        A, row_token, offsets, W, bias, out, E, N, K, a_rows, rows_ub, st, out_row, row_scale);
  }
}

// the weight layout of the shape picks the kernel; hp: H in 32-column blocks (slot order only)
template <int ACT, int OUT, bool GATHER>
hipError_t gemm(const moe_shape& s, const void* A, const int32_t* row_token,
                const int32_t* offsets, const void* W, const void* bias, void* out, int N, int K,
                int a_rows, int64_t rows_ub, hipStream_t st, const int32_t* out_row = nullptr,
                const float* row_scale = nullptr, bool hp = false) {
  if (s.dtype != MOE_BF16) return hipErrorInvalidValue;
  const bool small = skinny(s, rows_ub);
  auto a = (const bf16_t*)A;
  auto w = (const bf16_t*)W;
  auto b = (const bf16_t*)bias;
  auto o = (bf16_t*)out;
  const bool packed_w = s.weight_layout == MOE_WEIGHTS_PACKED;
  if constexpr (OUT == kOutSlots) {
    if (hp && !small) {
      if (packed_w)
        return run_gemm<ACT, OUT, GATHER, true, true>(small, a, row_token, offsets, w, b, o,
                                                      s.n_experts, N, K, a_rows, rows_ub, st,
                                                      out_row, row_scale);
      return run_gemm<ACT, OUT, GATHER, false, true>(small, a, row_token, offsets, w, b, o,
                                                     s.n_experts, N, K, a_rows, rows_ub, st,
                                                     out_row, row_scale);
    }
  }
  if (packed_w)
    return run_gemm<ACT, OUT, GATHER, true>(small, a, row_token, offsets, w, b, o, s.n_experts, N,
                                            K, a_rows, rows_ub, st, out_row, row_scale);
  return run_gemm<ACT, OUT, GATHER, false>(small, a, row_token, offsets, w, b, o, s.n_experts, N,
                                           K, a_rows, rows_ub, st, out_row, row_scale);
}

}  // namespace

hipError_t launch_ffn_up(const moe_shape& s, const void* x, const int32_t* row_token,
                         const int32_t* offsets, const void* w1, const void* b1, void* h,
                         int64_t rows_ub, hipStream_t st) {
  if (s.dtype != MOE_BF16)
    return launch_ffn_up_f32(s, x, row_token, offsets, w1, b1, h, rows_ub, st);
  return gemm<kActSilu, kOutSlots, true>(s, x, row_token, offsets, w1, b1, h, s.d_ff, s.d_model,
                                         (int)s.T, rows_ub, st, nullptr, nullptr,
                                         h_packed(s, rows_ub));
}

hipError_t launch_ffn_down(const moe_shape& s, const void* h, const int32_t* offsets,
                           const void* w2, const void* b2, void* y, int64_t rows_ub,
                           hipStream_t st) {
  if (s.dtype != MOE_BF16) return launch_ffn_down_f32(s, h, offsets, w2, b2, y, rows_ub, st);
  return gemm<kActNone, kOutSlots, false>(s, h, nullptr, offsets, w2, b2, y, s.d_model, s.d_ff,
                                          (int)rows_ub, rows_ub, st, nullptr, nullptr,
                                          h_packed(s, rows_ub));
}

// Gated expert (fused-MoE flow diagram, GEMM 1 -> SiLU x mul -> GEMM 2): GEMM 1 over the
// [2 d_ff, d_model] weights of each expert, gate rows first, with SiLU(gate) * up fused into
// the epilogue; no biases.  Output H: rows x d_ff in slot order (32-column blocks, see h_packed).
hipError_t launch_ffn_up_gated(const moe_shape& s, const void* x, const int32_t* row_token,
                               const int32_t* offsets, const void* w13, void* h, int64_t rows_ub,
                               hipStream_t st) {
  return gemm<kActGated, kOutSlots, true>(s, x, row_token, offsets, w13, nullptr, h, s.d_ff,
                                          s.d_model, (int)s.T, rows_ub, st, nullptr, nullptr,
                                          h_packed(s, rows_ub));
}

// GEMM 2 without bias (gated expert): Y = H W2^T
hipError_t launch_ffn_down_nobias(const moe_shape& s, const void* h, const int32_t* offsets,
                                  const void* w2, void* y, int64_t rows_ub, hipStream_t st) {
  return gemm<kActNone, kOutSlots, false>(s, h, nullptr, offsets, w2, nullptr, y, s.d_model,
                                          s.d_ff, (int)rows_ub, rows_ub, st, nullptr, nullptr,
                                          h_packed(s, rows_ub));
}

// ---------------------------------------------------------------- dropless pair order
// Fused-MoE flow diagram (moe-vllm flow): GEMM 1 reads token row p // top_k and writes pair row
// p; GEMM 2 reads pair row p and writes pair row p times topk_weights[p].  Both walk the pairs
// grouped by expert (sorted_pairs, expert e's at offsets[e] .. offsets[e+1] - 1), so each tile
// uses one expert's weights; row_token[i] = sorted_pairs[i] / top_k.  The tiles, the K order and
// so every product are those of the slot-order GEMMs; only where a row is read and written
// changes, and GEMM 2 multiplies by the pair's weight before the bf16 rounding.
hipError_t launch_ffn_up_pairs(const moe_shape& s, const void* x, const int32_t* row_token,
                               const int32_t* sorted_pairs, const int32_t* offsets,
                               const void* w1, const void* b1, void* h, int64_t rows_ub,
                               bool gated, hipStream_t st) {
  if (gated)
    return gemm<kActGated, kOutPairs, true>(s, x, row_token, offsets, w1, nullptr, h, s.d_ff,
                                            s.d_model, (int)s.T, rows_ub, st, sorted_pairs);
  return gemm<kActSilu, kOutPairs, true>(s, x, row_token, offsets, w1, b1, h, s.d_ff, s.d_model,
                                         (int)s.T, rows_ub, st, sorted_pairs);
}

// h and y hold T * top_k pair rows; b2 may be NULL (gated expert)
hipError_t launch_ffn_down_pairs(const moe_shape& s, const void* h, const int32_t* sorted_pairs,
                                 const int32_t* offsets, const void* w2, const void* b2,
                                 const float* weights, void* y, int64_t rows_ub, hipStream_t st) {
  return gemm<kActNone, kOutPairsScaled, true>(s, h, sorted_pairs, offsets, w2, b2, y, s.d_model,
                                               s.d_ff, (int)(s.T * s.top_k), rows_ub, st,
                                               sorted_pairs, weights);
}

}  // namespace moe
