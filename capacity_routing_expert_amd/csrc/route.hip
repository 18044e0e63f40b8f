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
// Mapping (gfx950): the logit GEMM [T, d] x [d, E] (E <= 256) is far too skinny and too
// precise for the bf16 matrix cores, but it fits the fp64 ones: one kernel reads x and the
// router weights once, multiplies them on v_mfma_f64_16x16x4f64 and finishes each block's
// tokens (bias, softmax, top-k) without a second launch or partial sums in memory.
#include "moe_internal.h"

namespace moe {

namespace {

// 8 bf16 (one 16-byte word) widened exactly to fp64
__device__ __forceinline__ void widen_bf16x8(uint4 q, double* v) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = (double)__uint_as_float(w[i] << 16);
    v[2 * i + 1] = (double)__uint_as_float(w[i] & 0xFFFF0000u);
  }
}

}  // namespace

// Bias, optional fp32 logits, softmax over all experts in fp64 (rounded once to fp32) and
// top-k for the TB tokens whose complete logits sit in lds[e * TB + i]; every thread of the
// block calls it, S = nthr / TB lanes per token (a power of two, inside one wave).
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

  // softmax + top-k: LPT = S lanes per token (a power of two, inside one wave);
  // lane `sub` owns experts e = sub (mod LPT)
  const int LPT = S;
  const int ti = threadIdx.x / LPT, sub = threadIdx.x % LPT;
  const int64_t tt = tok0 + ti;

  double m = -INFINITY;
  for (int e = sub; e < E; e += LPT) m = fmax(m, lds[e * TB + ti]);
  // lane exchanges: DPP moves for partners up to 8 lanes away, ds_bpermute beyond
  auto dxor = [](double v, int s) {
    return __longlong_as_double((long long)xor_partner((uint64_t)__double_as_longlong(v), s));
  };
  for (int off = LPT >> 1; off >= 1; off >>= 1) m = fmax(m, dxor(m, off));
  double z = 0.0;
  for (int e = sub; e < E; e += LPT) {
    const double v = exp(lds[e * TB + ti] - m);
    lds[e * TB + ti] = v;
    z += v;
  }
  for (int off = LPT >> 1; off >= 1; off >>= 1) z += dxor(z, off);
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
      const unsigned long long o = xor_partner(best, off);
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

// The same finish for at most 8 experts, without LDS round trips: 8 lanes per token, lane e
// (of an aligned group of 8) owns expert e.  The maximum, the sum of exponentials and each
// top-k round reduce over the 8 lanes with DPP lane moves in the order xor 4, 2, 1, which adds
// the same pairs as finish_group's butterfly over 16 lanes (its upper 8 lanes hold nothing), so
// both give the same bits.  bias_e is this lane's b_router entry, loaded by the caller early.
template <int TB>
__device__ void finish_e8(const double* lds, bool has_bias, float bias_e, int64_t tok0,
                          int64_t T, int E, int k, int nthr, int32_t* __restrict__ ids,
                          float* __restrict__ gates, float* __restrict__ logits_out) {
  const int e = threadIdx.x & 7;
  const bool ok = e < E;
  auto dxor = [](double v, int s) {
    return __longlong_as_double((long long)xor_partner((uint64_t)__double_as_longlong(v), s));
  };
  for (int base = 0; base < TB * 8; base += nthr) {  // whole waves leave together
    const int ti = (base + (int)threadIdx.x) >> 3;
    if (ti >= TB) break;
    const int64_t tt = tok0 + ti;
    double L = ok ? lds[e * TB + ti] : -INFINITY;
    if (ok && has_bias) L += (double)bias_e;
    if (ok && logits_out && tt < T) logits_out[tt * E + e] = (float)L;
    double m = L;
    for (int s = 4; s >= 1; s >>= 1) m = fmax(m, dxor(m, s));
    const double v = ok ? exp(L - m) : 0.0;
    double z = v;
    for (int s = 4; s >= 1; s >>= 1) z += dxor(z, s);
    // (gate descending, expert ascending) keys, as in finish_group; a taken expert's key is 0
    const float gv = (float)(v / z);
    uint64_t key = ok ? ((uint64_t)__float_as_uint(gv) << 32) | (0xFFFFFFFFull - (unsigned)e) : 0ull;
    for (int c = 0; c < k; ++c) {
      uint64_t best = key;
      for (int s = 4; s >= 1; s >>= 1) {
        const uint64_t o = xor_partner(best, s);
        best = o > best ? o : best;
      }
      const int ew = (int)(0xFFFFFFFFull - (best & 0xFFFFFFFFull));
      if (e == ew) key = 0ull;
      if (e == 0 && tt < T) {
        ids[tt * k + c] = ew;
        gates[tt * k + c] = __uint_as_float((uint32_t)(best >> 32));
      }
    }
  }
}

// ---------------------------------------------------------------- matrix-core router
// The logit GEMM [T, d] x [d, E] on the fp64 matrix cores: v_mfma_f64_16x16x4f64 multiplies a
// 16 x 4 tile of tokens by a 4 x 16 tile of experts, fp64 products of the widened inputs
// (exact) accumulated in fp64.  Both operands come from VGPRs, loaded straight from x and the
// router weights in the operand layout (lane l: token / expert l % 16, 8 consecutive columns of
// chunk 4 cq + l / 16), so every loaded value feeds 16 products and no weight table is needed.
// MFMA step s of chunk quad cq pairs column 8 (4 cq + l / 16) + s of both operands: a
// permutation of the summation order only.  A block of NW waves takes TT = 16 R tokens; wave w
// takes chunk quads w, w + NW, ...; wave 0 adds the other waves' partial tiles in wave order,
// so the logits are reproducible, then the block finishes its tokens (bias, softmax, top-k).
typedef double f64x4_t __attribute__((ext_vector_type(4)));

template <typename TIn>
struct Chunk8;
// The loads go through buffer resources over the whole matrix: a guarded-off chunk reads zeros
// from an out-of-range offset instead of sitting in a branch, so the compiler can count the
// loads in flight and wait only for the ones it needs (a predicated load made it wait for all).
template <>
struct Chunk8<bf16_t> {  // 8 bf16 columns as one 16-byte load (d % 8 == 0 for bf16)
  uint4 v;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t m, bool ok, int64_t row, int c,
                                       int d) {
    v = buffer_load16(m, ok && c * 8 < d ? (uint32_t)((row * d + (int64_t)c * 8) * 2) : kBufferOOR);
  }
  __device__ __forceinline__ void widen(double* o) const { widen_bf16x8(v, o); }
};
template <>
struct Chunk8<float> {  // 8 fp32 columns, each guarded (any d)
  float v[8];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t m, bool ok, int64_t row, int c,
                                       int d) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int col = c * 8 + u;
      v[u] = buffer_load_f32(m, ok && col < d ? (uint32_t)((row * d + col) * 4) : kBufferOOR);
    }
  }
  __device__ __forceinline__ void widen(double* o) const {
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = v[u];
  }
};

template <typename TIn, int R, int EBG, int NW, int PF>
__global__ __launch_bounds__(64 * NW) void k_route_mfma(
    const TIn* __restrict__ x, const TIn* __restrict__ w, const float* __restrict__ b_router,
    int64_t T, int d, int E, int k, int32_t* __restrict__ ids, float* __restrict__ gates,
    float* __restrict__ logits_out) {
  constexpr int TT = 16 * R, NT = 64 * NW;
  constexpr int kPart = R * EBG * 256;  // doubles in one wave's partial tiles
  extern __shared__ double lds[];       // [NW - 1][kPart] partials, then logits [E][TT]
  double* logit = lds + (NW - 1) * kPart;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, q = lane >> 4;
  const int64_t tok0 = (int64_t)blockIdx.x * TT;
  const int d8 = (d + 7) / 8, nq = (d8 + 3) / 4;
  const int EB = (E + 15) / 16;
  // x and the router weights (< 2 GiB each, host-checked)
  const __amdgpu_buffer_rsrc_t xs = buffer_rsrc(x, (uint32_t)(T * d * (int64_t)sizeof(TIn)));
  const __amdgpu_buffer_rsrc_t ws = buffer_rsrc(w, (uint32_t)((int64_t)E * d * sizeof(TIn)));

  // with a single 16 x 16 tile per wave, even and odd MFMA steps go to two accumulators, so
  // consecutive MFMAs do not wait on each other (the two are added at the end: a permutation of
  // the summation order only)
  constexpr int NACC = R * EBG == 1 ? 2 : 1;
  for (int b0 = 0; b0 < EB; b0 += EBG) {
    f64x4_t accs[NACC][R][EBG];
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int bb = 0; bb < EBG; ++bb) accs[a][r][bb] = f64x4_t{0.0, 0.0, 0.0, 0.0};

    // wave w takes chunk quads w, w + NW, ... in that order, with PF quads in flight: the raw
    // loads of quad cq + PF NW are issued as soon as quad cq is widened (quads past the end
    // load zeros, whose exact zero products leave the sums as they are)
    Chunk8<TIn> xr[PF][R], wr[PF][EBG];
    auto load = [&](int p, int cq) {
      const int c = cq * 4 + q;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t t = tok0 + 16 * r + i;
        xr[p][r].load(xs, cq < nq && t < T, t, c, d);
      }
#pragma unroll
      for (int bb = 0; bb < EBG; ++bb) {
        const int e = (b0 + bb) * 16 + i;
        wr[p][bb].load(ws, cq < nq && e < E, e, c, d);
      }
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) load(p, wave + p * NW);
    for (int cq0 = wave; cq0 < nq; cq0 += PF * NW) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        double xa[R][8], wb[EBG][8];
#pragma unroll
        for (int r = 0; r < R; ++r) xr[p][r].widen(xa[r]);
#pragma unroll
        for (int bb = 0; bb < EBG; ++bb) wr[p][bb].widen(wb[bb]);
        load(p, cq0 + (p + PF) * NW);
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8)
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int bb = 0; bb < EBG; ++bb)
              accs[s8 % NACC][r][bb] = __builtin_amdgcn_mfma_f64_16x16x4f64(
                  xa[r][s8], wb[bb][s8], accs[s8 % NACC][r][bb], 0, 0, 0);
      }
    }

    auto& acc = accs[0];
    if constexpr (NACC == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[0][0][j] += accs[1][0][0][j];
    }
    // lane l, register j of a tile holds token 4 j + l / 16, expert l % 16 of the tile
    if (wave > 0) {
      double* mine = lds + (wave - 1) * kPart;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int bb = 0; bb < EBG; ++bb)
#pragma unroll
          for (int j = 0; j < 4; ++j) mine[((r * EBG + bb) * 64 + lane) * 4 + j] = acc[r][bb][j];
    }
    __syncthreads();
    if (wave == 0) {
      for (int ww = 1; ww < NW; ++ww) {
        const double* other = lds + (ww - 1) * kPart;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int bb = 0; bb < EBG; ++bb)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[r][bb][j] += other[((r * EBG + bb) * 64 + lane) * 4 + j];
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int bb = 0; bb < EBG; ++bb) {
          const int e = (b0 + bb) * 16 + i;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (e < E) logit[e * TT + 16 * r + 4 * j + q] = acc[r][bb][j];
        }
    }
    __syncthreads();
  }
  finish_group<TT>(logit, b_router, tok0, T, E, k, NT / TT, NT, ids, gates, logits_out);
}

// dynamic LDS of the largest router block: 7 wave partials of 2 expert tiles + [256][16] logits
constexpr size_t route_lds_max() { return (size_t)8 * (7 * 2 * 256 + 256 * 16); }

// ---------------------------------------------------------------- matrix-core router, E <= 8
// With at most 8 experts a 16 x 16 tile is half padding.  v_mfma_f64_4x4x4f64 runs four
// independent 4 x 4 x 4 products per instruction at the full fp64 matrix rate (probe, 8 waves
// per SIMD: 77 TFLOP/s, against 73 for the 16 x 16 x 4 instruction).  Its lane layout (probe):
// lane l = 16 g + 4 b + r holds row r of block b's A operand and column r of block b's B operand
// at step g of the 4-deep contraction, and receives row g, column r of block b's result.
// The four blocks take four groups of 4 tokens (block b: tokens 4 b .. 4 b + 3 of a 16-token
// row group) and the same 4 experts, and two instructions per step cover experts 0 .. 3 and
// 4 .. 7.  So every lane loads x chunks that no other lane loads (only the small router weights
// are loaded by several lanes), and a wave's 16 x 8 tile has no padding.  As in k_route_mfma,
// lane l loads 8 consecutive columns of its token and of its expert (chunk 4 cq + g), and MFMA
// step s pairs column s of both: a permutation of the summation order only.  A block of NW
// waves takes TT = 16 RT tokens, wave w takes chunk quads w, w + NW, ..., and wave 0 adds the
// other waves' partial tiles in wave order before the block finishes its tokens.  Each block
// starts its walk over those quads at its own point (block index modulo the quad count) and
// wraps around, so that the blocks do not all read the same columns of x at once (a fixed
// order per block: the logits are still reproducible).
template <typename TIn, int RT, int NW, int PF>
__global__ __launch_bounds__(64 * NW) void k_route_mfma4(
    const TIn* __restrict__ x, const TIn* __restrict__ w, const float* __restrict__ b_router,
    int64_t T, int d, int E, int k, int32_t* __restrict__ ids, float* __restrict__ gates,
    float* __restrict__ logits_out) {
  constexpr int TT = 16 * RT, NT = 64 * NW;
  __shared__ double part[NW > 1 ? NW - 1 : 1][2 * RT][64];  // waves 1 .. NW - 1: partial tiles
  __shared__ double logit[8 * TT];                          // [expert][token of the block]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, b = (lane >> 2) & 3, r = lane & 3;
  const int64_t tok0 = (int64_t)blockIdx.x * TT;
  const int d8 = (d + 7) / 8, nq = (d8 + 3) / 4;
  // x and the router weights (< 2 GiB each, host-checked)
  const __amdgpu_buffer_rsrc_t xs = buffer_rsrc(x, (uint32_t)(T * d * (int64_t)sizeof(TIn)));
  const __amdgpu_buffer_rsrc_t ws = buffer_rsrc(w, (uint32_t)((int64_t)E * d * sizeof(TIn)));

  // acc[eg][rr]: experts 4 eg .. 4 eg + 3 of row group rr (the two expert groups alternate, so
  // consecutive MFMAs do not wait on each other)
  double acc[2][RT];
#pragma unroll
  for (int eg = 0; eg < 2; ++eg)
#pragma unroll
    for (int rr = 0; rr < RT; ++rr) acc[eg][rr] = 0.0;
  Chunk8<TIn> xr[PF][RT], wr[PF][2];
  auto load = [&](int p, int cq) {
    const int c = cq * 4 + g;
#pragma unroll
    for (int rr = 0; rr < RT; ++rr) {
      const int64_t t = tok0 + 16 * rr + 4 * b + r;
      xr[p][rr].load(xs, cq < nq && t < T, t, c, d);
    }
#pragma unroll
    for (int eg = 0; eg < 2; ++eg) {
      const int e = 4 * eg + r;
      wr[p][eg].load(ws, cq < nq && e < E, e, c, d);
    }
  };
  // this wave's n_w quads wave, wave + NW, ..., walked from index j0 on; indices past n_w give
  // quad nq, whose loads read zeros
  const int n_w = wave < nq ? (nq - wave + NW - 1) / NW : 0;
  const int j0 = n_w ? (int)(blockIdx.x % (unsigned)n_w) : 0;
  auto quad_of = [&](int i) { return i < n_w ? wave + NW * ((j0 + i) % n_w) : nq; };
#pragma unroll
  for (int p = 0; p < PF; ++p) load(p, quad_of(p));
  // this lane's router bias for the finish, loaded behind the first quads (the waits for those
  // then do not include it)
  const float bias_e =
      b_router && (int)(threadIdx.x & 7) < E ? b_router[threadIdx.x & 7] : 0.0f;
  for (int i0 = 0; i0 < n_w; i0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      double xa[RT][8], wb[2][8];
#pragma unroll
      for (int rr = 0; rr < RT; ++rr) xr[p][rr].widen(xa[rr]);
      wr[p][0].widen(wb[0]);
      wr[p][1].widen(wb[1]);
      load(p, quad_of(i0 + p + PF));
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8)
#pragma unroll
        for (int rr = 0; rr < RT; ++rr)
#pragma unroll
          for (int eg = 0; eg < 2; ++eg)
            acc[eg][rr] =
                __builtin_amdgcn_mfma_f64_4x4x4f64(xa[rr][s8], wb[eg][s8], acc[eg][rr], 0, 0, 0);
    }
  }
  // lane l holds token 16 rr + 4 b + g of the block, expert 4 eg + r
  if (wave > 0) {
#pragma unroll
    for (int eg = 0; eg < 2; ++eg)
#pragma unroll
      for (int rr = 0; rr < RT; ++rr) part[wave - 1][eg * RT + rr][lane] = acc[eg][rr];
  }
  __syncthreads();
  if (wave == 0) {
    for (int ww = 1; ww < NW; ++ww)
#pragma unroll
      for (int eg = 0; eg < 2; ++eg)
#pragma unroll
        for (int rr = 0; rr < RT; ++rr) acc[eg][rr] += part[ww - 1][eg * RT + rr][lane];
#pragma unroll
    for (int eg = 0; eg < 2; ++eg) {
      const int e = 4 * eg + r;
#pragma unroll
      for (int rr = 0; rr < RT; ++rr)
        if (e < E) logit[e * TT + 16 * rr + 4 * b + g] = acc[eg][rr];
    }
  }
  __syncthreads();
  finish_e8<TT>(logit, b_router != nullptr, bias_e, tok0, T, E, k, NT, ids, gates, logits_out);
}

// The same 16-token x 8-expert tile with the four blocks of v_mfma_f64_4x4x4f64 on four
// slices of d instead of four token groups.  Block b's 4 x 4 product then takes tokens 4 tg ..
// 4 tg + 3 and experts 4 eg .. 4 eg + 3 (one instruction per token group tg and expert group eg)
// over the columns of slice b, and lane l = 16 g + 4 b + r loads chunk 16 cq + 4 b + g of token
// 4 tg + r and of expert 4 eg + r.  No two lanes load or widen the same router weights (in
// k_route_mfma4 the four blocks share them: twice as many widenings per product), and a wave
// covers 128 columns per chunk quad.  MFMA step s pairs column s of both chunks, as there.  Lane
// (g, b, r) ends with slice b's partial logit of token 4 tg + g, expert 4 eg + r; the four slices
// are added over the lanes b = 0 .. 3 (xor 4, then xor 8: every lane of the four gets the same
// sum), then the waves' tiles in wave order.  Only the summation order differs from
// k_route_mfma4.
template <typename TIn, int NW, int PF>
__global__ __launch_bounds__(64 * NW) void k_route_mfma4k(
    const TIn* __restrict__ x, const TIn* __restrict__ w, const float* __restrict__ b_router,
    int64_t T, int d, int E, int k, int32_t* __restrict__ ids, float* __restrict__ gates,
    float* __restrict__ logits_out) {
  constexpr int TT = 16, NT = 64 * NW;
  __shared__ double part[NW > 1 ? NW - 1 : 1][8][64];  // waves 1 .. NW - 1: partial tiles
  __shared__ double logit[8 * TT];                     // [expert][token of the block]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, b = (lane >> 2) & 3, r = lane & 3;
  const int64_t tok0 = (int64_t)blockIdx.x * TT;
  const int d8 = (d + 7) / 8, nq = (d8 + 15) / 16;
  const __amdgpu_buffer_rsrc_t xs = buffer_rsrc(x, (uint32_t)(T * d * (int64_t)sizeof(TIn)));
  const __amdgpu_buffer_rsrc_t ws = buffer_rsrc(w, (uint32_t)((int64_t)E * d * sizeof(TIn)));

  double acc[4][2];  // [token group][expert group]
#pragma unroll
  for (int tg = 0; tg < 4; ++tg) acc[tg][0] = acc[tg][1] = 0.0;
  Chunk8<TIn> xr[PF][4], wr[PF][2];
  auto load = [&](int p, int cq) {
    const int c = cq * 16 + b * 4 + g;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const int64_t t = tok0 + 4 * tg + r;
      xr[p][tg].load(xs, cq < nq && t < T, t, c, d);
    }
#pragma unroll
    for (int eg = 0; eg < 2; ++eg) {
      const int e = 4 * eg + r;
      wr[p][eg].load(ws, cq < nq && e < E, e, c, d);
    }
  };
  // this wave's n_w quads wave, wave + NW, ..., walked from a per-block point on (as in
  // k_route_mfma4); indices past n_w give quad nq, whose loads read zeros
  const int n_w = wave < nq ? (nq - wave + NW - 1) / NW : 0;
  const int j0 = n_w ? (int)(blockIdx.x % (unsigned)n_w) : 0;
  auto quad_of = [&](int i) { return i < n_w ? wave + NW * ((j0 + i) % n_w) : nq; };
#pragma unroll
  for (int p = 0; p < PF; ++p) load(p, quad_of(p));
  const float bias_e =
      b_router && (int)(threadIdx.x & 7) < E ? b_router[threadIdx.x & 7] : 0.0f;
  for (int i0 = 0; i0 < n_w; i0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      double xa[4][8], wb[2][8];
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) xr[p][tg].widen(xa[tg]);
      wr[p][0].widen(wb[0]);
      wr[p][1].widen(wb[1]);
      load(p, quad_of(i0 + p + PF));
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8)
#pragma unroll
        for (int tg = 0; tg < 4; ++tg)
#pragma unroll
          for (int eg = 0; eg < 2; ++eg)
            acc[tg][eg] =
                __builtin_amdgcn_mfma_f64_4x4x4f64(xa[tg][s8], wb[eg][s8], acc[tg][eg], 0, 0, 0);
    }
  }
  // slices: lanes b = 0 .. 3 of (g, r)
  auto dxor = [](double v, int st) {
    return __longlong_as_double((long long)xor_partner((uint64_t)__double_as_longlong(v), st));
  };
#pragma unroll
  for (int tg = 0; tg < 4; ++tg)
#pragma unroll
    for (int eg = 0; eg < 2; ++eg) {
      acc[tg][eg] += dxor(acc[tg][eg], 4);
      acc[tg][eg] += dxor(acc[tg][eg], 8);
    }
  if (wave > 0) {
#pragma unroll
    for (int tg = 0; tg < 4; ++tg)
#pragma unroll
      for (int eg = 0; eg < 2; ++eg) part[wave - 1][tg * 2 + eg][lane] = acc[tg][eg];
  }
  __syncthreads();
  if (wave == 0) {
    for (int ww = 1; ww < NW; ++ww)
#pragma unroll
      for (int tg = 0; tg < 4; ++tg)
#pragma unroll
        for (int eg = 0; eg < 2; ++eg) acc[tg][eg] += part[ww - 1][tg * 2 + eg][lane];
    if (b == 0) {
#pragma unroll
      for (int eg = 0; eg < 2; ++eg) {
        const int e = 4 * eg + r;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg)
          if (e < E) logit[e * TT + 4 * tg + g] = acc[tg][eg];
      }
    }
  }
  __syncthreads();
  finish_e8<TT>(logit, b_router != nullptr, bias_e, tok0, T, E, k, NT, ids, gates, logits_out);
}

namespace {

template <typename TIn, int EBG, int NW>
hipError_t route_launch(const moe_shape& s, const TIn* x, const TIn* w, const float* b_router,
                        int32_t* ids, float* gates, float* logits, hipStream_t st) {
  constexpr int R = 1, TT = 16 * R;
  // chunk quads in flight per wave besides the one being multiplied: with branch-free loads one
  // is enough (4 and 8 measured no faster, and 8 slower on the large layers)
  constexpr int PF = 1;
  const size_t lds = (size_t)8 * ((NW - 1) * R * EBG * 256 + (size_t)s.n_experts * TT);
  auto kern = k_route_mfma<TIn, R, EBG, NW, PF>;
  static std::atomic<bool> lds_allowed[kMaxDevices];
  if (hipError_t err = allow_dynamic_lds((const void*)kern, (int)route_lds_max(), lds_allowed);
      err != hipSuccess)
    return err;
  const int64_t blocks = (s.T + TT - 1) / TT;
  return launch_timed(kern, dim3((unsigned)blocks), dim3(64 * NW), lds, st, x, w, b_router, s.T,
                      s.d_model, s.n_experts, s.top_k, ids, gates, logits);
}

// Tile plan: 16 tokens per block; one or two tiles of 16 experts per pass over x, more experts
// take more passes (the block's x rows come back from L2).  Two tiles need about 120 VGPRs, so
// several blocks share a CU and one block's cross-wave sum and softmax overlap another's MFMAs
// (four tiles per pass, 252 VGPRs and one block per CU, ran the 64-expert fine layer's router
// at 118 us against 97 us).  Batches of at least 8192 tokens (two blocks or more per CU) use
// 4-wave blocks, which fit more blocks per CU (fine 104 -> 95 us); smaller ones use 8 waves,
// which shortens each wave's walk over d (decode 10.7 -> 10.4 us).
template <typename TIn, int EBG>
hipError_t route_waves(const moe_shape& s, const TIn* x, const TIn* w, const float* b_router,
                       int32_t* ids, float* gates, float* logits, hipStream_t st) {
  if (s.T >= 8192) return route_launch<TIn, EBG, 4>(s, x, w, b_router, ids, gates, logits, st);
  return route_launch<TIn, EBG, 8>(s, x, w, b_router, ids, gates, logits, st);
}

template <typename TIn, int RT, int NW>
hipError_t route4_launch(const moe_shape& s, const TIn* x, const TIn* w, const float* b_router,
                         int32_t* ids, float* gates, float* logits, hipStream_t st) {
  constexpr int TT = 16 * RT, PF = 2;
  return launch_timed(k_route_mfma4<TIn, RT, NW, PF>, dim3((unsigned)((s.T + TT - 1) / TT)),
                      dim3(64 * NW), 0, st, x, w, b_router, s.T, s.d_model, s.n_experts,
                      s.top_k, ids, gates, logits);
}

template <typename TIn>
hipError_t route_any(const moe_shape& s, const TIn* x, const TIn* w, const float* b_router,
                     int32_t* ids, float* gates, float* logits, hipStream_t st) {
  // At most 8 experts: 16-token x 8-expert tiles, 4-wave blocks, two chunk quads in flight per
  // wave.  From 16384 tokens a lane takes 4 row groups (64 tokens per block: the weight loads
  // and widenings are shared by more tiles); smaller batches take 16 tokens per block (more
  // blocks) with the four MFMA blocks on four slices of d, so that no two lanes widen the same
  // weights (k_route_mfma4k).  Lab, same routing: collapse layer 97 us with the 16 x 16 tiles,
  // 72 to 78 us with 8-token x 8-expert tiles (two lanes loading each x chunk), 56 us with these;
  // mid 13.0 -> 12.3 us.  Same-box stage times of the d slices against the token groups: mid
  // 13.6-13.8 -> 12.1-12.8 us, decode (64 tokens) 11.6-11.7 -> 9.6-9.9 us.
  if (s.n_experts <= 8) {
    if (s.T >= 16384) return route4_launch<TIn, 4, 4>(s, x, w, b_router, ids, gates, logits, st);
    constexpr int NW = 4, PF = 2;
    return launch_timed(k_route_mfma4k<TIn, NW, PF>, dim3((unsigned)((s.T + 15) / 16)),
                        dim3(64 * NW), 0, st, x, w, b_router, s.T, s.d_model, s.n_experts,
                        s.top_k, ids, gates, logits);
  }
  if (s.n_experts <= 16) return route_waves<TIn, 1>(s, x, w, b_router, ids, gates, logits, st);
  return route_waves<TIn, 2>(s, x, w, b_router, ids, gates, logits, st);
}

}  // namespace

hipError_t launch_route(const moe_shape& s, const void* x, const void* w_router,
                        const float* b_router, int32_t* ids, float* gates, float* logits,
                        hipStream_t st) {
  if (s.dtype == MOE_BF16)
    return route_any<bf16_t>(s, (const bf16_t*)x, (const bf16_t*)w_router, b_router, ids, gates,
                             logits, st);
  return route_any<float>(s, (const float*)x, (const float*)w_router, b_router, ids, gates,
                          logits, st);
}

}  // namespace moe
