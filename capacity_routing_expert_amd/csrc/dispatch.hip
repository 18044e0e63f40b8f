// Dispatch: per-expert counts, capacity cut and slot assignment.
//
// Worked Example (capacity paragraph): an expert receiving more tokens than its capacity
// keeps the most confident ones; the least confident is dropped and takes the residual
// path.  "Some Tokens Do Not Get In", "Past the edge": tokens claim slots of their expert's
// fixed buffer in some order until it is full.  Order used here, over every choice rank of
// every token together: gate descending, then token index ascending, then choice ascending.
// For an assignment i = t*k + c the last two keys are simply i ascending, so each expert's
// order is the ascending order of the 64-bit key (~ord(gate) << 32) | i, which is unique:
// any correct sort gives the same slots.
//
// Kernels (N = T*k assignments):
//   k_dispatch_hist    per block of kDispatchChunk assignments, an expert histogram built
//                      from wavefront ballots (lanes with equal expert id are matched
//                      with 9 ballots; one leader per group adds to an LDS counter);
//   k_dispatch_scatter every block sums the histograms of the blocks before it (bucket
//                      base), then scatters its keys stably into per-expert buckets using
//                      the same ballot match for the in-wave rank; block 0 publishes the
//                      counts, the kept-slot offsets and the bucket starts;
//   k_dispatch_rank    one block per kRankChunk keys of one expert bucket: bitonic sort in
//                      LDS; a bucket that fits one chunk has its ranks right there and emits
//                      slot_of / drop_mask / row_token; larger buckets write the sorted chunk;
//   k_dispatch_merge   only for buckets spanning several chunks: rank = position in own
//                      chunk + lower bounds in the bucket's other sorted chunks (staged
//                      through LDS), then emit.
// No floating-point atomics, no order-dependent reductions: the result is deterministic.
#include "moe_internal.h"

namespace moe {

namespace {

// Lanes of the wave holding the same `key` (0..511), restricted to lanes with `valid`.
__device__ __forceinline__ uint64_t match_key(int key, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 9; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    m &= bit ? bb : ~bb;
  }
  return valid ? m : 0ull;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// ascending order of the key <=> gate descending (-0 taken as +0), then assignment index
__device__ __forceinline__ uint64_t sort_key(float g, uint32_t i) {
  uint32_t u = __float_as_uint(g);
  if (u == 0x80000000u) u = 0u;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)(~ord) << 32) | (uint64_t)i;
}

// Exclusive scan of n ints in LDS by one wave; each lane reads and rewrites only its own
// contiguous range, the lanes exchange partial sums through shuffles.
__device__ void wave_exclusive_scan(int* a, int n, int* total_out) {
  const int lane = threadIdx.x & 63;
  const int per = (n + 63) / 64;
  const int b = lane * per;
  int s = 0;
  for (int j = 0; j < per; ++j)
    if (b + j < n) s += a[b + j];
  int inc = s;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  int run = inc - s;
  for (int j = 0; j < per; ++j)
    if (b + j < n) {
      const int v = a[b + j];
      a[b + j] = run;
      run += v;
    }
  if (total_out) *total_out = __shfl(inc, 63, 64);
}

}  // namespace

__global__ __launch_bounds__(256) void k_dispatch_hist(const int32_t* __restrict__ ids, int64_t N,
                                                       int E, int32_t* __restrict__ blk_hist) {
  __shared__ int cnt[260];
  for (int i = threadIdx.x; i <= E; i += 256) cnt[i] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kDispatchChunk;
  for (int r = 0; r < kDispatchChunk / 256; ++r) {
    const int64_t i = base + r * 256 + threadIdx.x;
    const bool valid = i < N;
    int e = valid ? ids[i] : 0;
    if (e < 0 || e >= E) e = E;  // out-of-range ids go to an overflow bucket
    const uint64_t peers = match_key(e, valid);
    if (valid && (peers & lanemask_lt()) == 0) atomicAdd(&cnt[e], __popcll(peers));
  }
  __syncthreads();
  for (int i = threadIdx.x; i <= E; i += 256) blk_hist[(int64_t)blockIdx.x * (E + 1) + i] = cnt[i];
}

__global__ __launch_bounds__(256) void k_dispatch_scatter(
    const int32_t* __restrict__ ids, const float* __restrict__ gates, int64_t N, int E, int cap,
    int nb, const int32_t* __restrict__ blk_hist, uint64_t* __restrict__ keys,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ seg_start,
    int32_t* __restrict__ slot_of, uint8_t* __restrict__ drop) {
  __shared__ int s_cnt[260], s_run[260], s_kept[260];
  __shared__ int wcnt[4][260];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e <= E; e += 256) {
    int tot = 0, pre = 0;
    for (int b = 0; b < nb; ++b) {
      const int h = blk_hist[(int64_t)b * (E + 1) + e];
      if (b < (int)blockIdx.x) pre += h;
      tot += h;
    }
    s_cnt[e] = tot;
    s_run[e] = pre;
    s_kept[e] = e < E ? min(tot, cap) : 0;
    for (int w = 0; w < 4; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid < E) counts[tid] = s_cnt[tid];
  __syncthreads();
  if (wave == 0) {
    wave_exclusive_scan(s_cnt, E + 1, nullptr);  // s_cnt becomes the bucket starts
    if (blockIdx.x == 0) wave_exclusive_scan(s_kept, E + 1, nullptr);
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = tid; e <= E; e += 256) {
      offsets[e] = s_kept[e];     // exclusive prefix of min(count, cap); offsets[E] = N_kept
      seg_start[e] = s_cnt[e];
    }
  }
  for (int e = tid; e <= E; e += 256) s_run[e] += s_cnt[e];
  __syncthreads();

  const int64_t base = (int64_t)blockIdx.x * kDispatchChunk;
  for (int r = 0; r < kDispatchChunk / 256; ++r) {
    const int64_t i = base + r * 256 + tid;
    const bool valid = i < N;
    int e = valid ? ids[i] : 0;
    if (e < 0 || e >= E) e = E;
    const uint64_t peers = match_key(e, valid);
    const int rank = __popcll(peers & lanemask_lt());
    if (valid && rank == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = s_run[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      if (e < E) {
        keys[pos] = sort_key(gates[i], (uint32_t)i);
      } else {
        keys[pos] = ~0ull;
        slot_of[i] = -1;
        drop[i] = 1;
      }
    }
    __syncthreads();
    for (int ee = tid; ee <= E; ee += 256) {
      s_run[ee] += wcnt[0][ee] + wcnt[1][ee] + wcnt[2][ee] + wcnt[3][ee];
      wcnt[0][ee] = wcnt[1][ee] = wcnt[2][ee] = wcnt[3][ee] = 0;
    }
    __syncthreads();
  }
}

namespace {

constexpr int kRankThreads = 512;

// Which (expert, chunk) this block serves; returns false if the block has no chunk.
// Called by every thread of the block (contains barriers).
__device__ bool find_chunk(const int32_t* __restrict__ counts, int E, int* s_pref, int* out_e,
                           int* out_j) {
  __shared__ int s_e, s_j, s_ok;
  for (int e = threadIdx.x; e <= E; e += blockDim.x)
    s_pref[e] = e < E ? (counts[e] + kRankChunk - 1) / kRankChunk : 0;
  __syncthreads();
  if ((threadIdx.x >> 6) == 0) wave_exclusive_scan(s_pref, E + 1, nullptr);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int b = blockIdx.x;
    s_ok = 0;
    for (int e = 0; e < E; ++e) {
      if (b >= s_pref[e] && b < s_pref[e + 1]) {
        s_e = e;
        s_j = b - s_pref[e];
        s_ok = 1;
        break;
      }
    }
  }
  __syncthreads();
  *out_e = s_e;
  *out_j = s_j;
  return s_ok != 0;
}

__device__ void bitonic_sort(uint64_t* a, int P) {
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int idx = threadIdx.x; idx < (P >> 1); idx += kRankThreads) {
        const int lo = 2 * idx - (idx & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t x = a[lo], y = a[hi];
        if ((x > y) == up) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ void emit(uint64_t key, int r, int e, int k, int cap,
                                     const int32_t* __restrict__ offsets,
                                     int32_t* __restrict__ slot_of, int32_t* __restrict__ row_token,
                                     uint8_t* __restrict__ drop) {
  const uint32_t i = (uint32_t)(key & 0xFFFFFFFFull);
  if (r < cap) {
    const int s = offsets[e] + r;
    slot_of[i] = s;
    drop[i] = 0;
    row_token[s] = (int32_t)(i / (uint32_t)k);
  } else {
    slot_of[i] = -1;
    drop[i] = 1;
  }
}

}  // namespace

__global__ __launch_bounds__(kRankThreads) void k_dispatch_rank(
    uint64_t* __restrict__ keys, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ seg_start, int E, int k,
    int cap, int32_t* __restrict__ slot_of, int32_t* __restrict__ row_token,
    uint8_t* __restrict__ drop) {
  __shared__ uint64_t sk[kRankChunk];
  __shared__ int s_pref[260];
  int e, j;
  if (!find_chunk(counts, E, s_pref, &e, &j)) return;
  const int n = counts[e];
  const int64_t start = (int64_t)seg_start[e] + (int64_t)j * kRankChunk;
  const int m = min(kRankChunk, n - j * kRankChunk);
  int P = 64;
  while (P < m) P <<= 1;
  for (int p = threadIdx.x; p < P; p += kRankThreads) sk[p] = p < m ? keys[start + p] : ~0ull;
  __syncthreads();
  bitonic_sort(sk, P);
  if (n <= kRankChunk) {
    for (int p = threadIdx.x; p < m; p += kRankThreads)
      emit(sk[p], p, e, k, cap, offsets, slot_of, row_token, drop);
  } else {
    for (int p = threadIdx.x; p < m; p += kRankThreads) keys[start + p] = sk[p];
  }
}

__global__ __launch_bounds__(kRankThreads) void k_dispatch_merge(
    const uint64_t* __restrict__ keys, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ seg_start, int E, int k,
    int cap, int32_t* __restrict__ slot_of, int32_t* __restrict__ row_token,
    uint8_t* __restrict__ drop) {
  __shared__ uint64_t sk[kRankChunk];
  __shared__ int s_pref[260];
  constexpr int PER = kRankChunk / kRankThreads;
  int e, j;
  if (!find_chunk(counts, E, s_pref, &e, &j)) return;
  const int n = counts[e];
  if (n <= kRankChunk) return;
  const int nch = (n + kRankChunk - 1) / kRankChunk;
  const int64_t seg = seg_start[e];
  const int m = min(kRankChunk, n - j * kRankChunk);
  uint64_t mine[PER];
  int rank[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int p = threadIdx.x + u * kRankThreads;
    mine[u] = p < m ? keys[seg + (int64_t)j * kRankChunk + p] : ~0ull;
    rank[u] = p;
  }
  for (int jj = 0; jj < nch; ++jj) {
    if (jj == j) continue;
    const int mm = min(kRankChunk, n - jj * kRankChunk);
    __syncthreads();
    for (int p = threadIdx.x; p < mm; p += kRankThreads) sk[p] = keys[seg + (int64_t)jj * kRankChunk + p];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      int lo = 0, hi = mm;  // first position with sk[pos] >= mine (keys are unique)
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sk[mid] < mine[u]) lo = mid + 1; else hi = mid;
      }
      rank[u] += lo;
    }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int p = threadIdx.x + u * kRankThreads;
    if (p < m) emit(mine[u], rank[u], e, k, cap, offsets, slot_of, row_token, drop);
  }
}

hipError_t launch_dispatch(const moe_shape& s, const int32_t* ids, const float* gates,
                           int32_t* counts, int32_t* offsets, int32_t* slot_of,
                           int32_t* row_token, uint8_t* drop, int32_t* seg_start,
                           int32_t* blk_hist, uint64_t* keys, hipStream_t st) {
  const int64_t N = s.T * (int64_t)s.top_k;
  const int E = s.n_experts;
  const int nb = (int)((N + kDispatchChunk - 1) / kDispatchChunk);
  hipLaunchKernelGGL(k_dispatch_hist, dim3(nb), dim3(256), 0, st, ids, N, E, blk_hist);
  hipLaunchKernelGGL(k_dispatch_scatter, dim3(nb), dim3(256), 0, st, ids, gates, N, E, s.capacity,
                     nb, blk_hist, keys, counts, offsets, seg_start, slot_of, drop);
  const int grid = (int)((N + kRankChunk - 1) / kRankChunk) + E;
  hipLaunchKernelGGL(k_dispatch_rank, dim3(grid), dim3(kRankThreads), 0, st, keys, counts, offsets,
                     seg_start, E, s.top_k, s.capacity, slot_of, row_token, drop);
  hipLaunchKernelGGL(k_dispatch_merge, dim3(grid), dim3(kRankThreads), 0, st, keys, counts,
                     offsets, seg_start, E, s.top_k, s.capacity, slot_of, row_token, drop);
  return hipGetLastError();
}

}  // namespace moe
