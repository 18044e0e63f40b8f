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
//   k_dispatch_hist    per block of `chunk` assignments, an expert histogram built
//                      from wavefront ballots (lanes with equal expert id are matched
//                      with 9 ballots; one leader per group adds to an LDS counter);
//   k_dispatch_scatter every block sums the histograms of the blocks before it (bucket
//                      base), then scatters its keys stably into per-expert buckets using
//                      the same ballot match for the in-wave rank; block 0 publishes the
//                      counts, the kept-slot offsets and the bucket starts;
//   k_dispatch_tilesort each 256-key tile of a bucket is sorted in LDS (bitonic network);
//   k_dispatch_rank    rank of a key = number of smaller keys of its bucket: its position in
//                      its own sorted tile plus a binary search in every other tile of the
//                      bucket; blocks take (tile, group of 4 other tiles) work items and add
//                      their partial counts with integer atomics (exact and order-free);
//   k_dispatch_emit    slot_of / drop_mask / row_token from the ranks and the capacity.
// Up to 1024 assignments a single workgroup does all of it instead (k_dispatch_small: one
// bitonic sort of the (expert, fill order) keys, one per thread), which saves four dependent
// launches.  Up to 16384 assignments two launches do it: runs of 512 keys sorted in LDS
// (k_dispatch_runs), then every key ranked against all runs held in one workgroup's LDS and its
// slot written (k_dispatch_merge).
// Integer results only, no order-dependent reductions: the output is deterministic.
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

// (expert, fill order) key of assignment i < 2^24 with expert e in [0, E): ascending order is the
// expert, then gate descending, then i ascending
__device__ __forceinline__ uint64_t expert_key(int e, float g, uint32_t i) {
  return ((uint64_t)e << 56) | ((sort_key(g, 0u) >> 32) << 24) | (uint64_t)i;
}
// key of an assignment i whose id lies outside [0, E): kInvalidKey | i sorts after every valid
// key (~ord(gate) < 0xFFFFFFFF for any non-NaN gate), and padding (~0) after both
constexpr uint64_t kInvalidKey = 0xFFFFFFFFFF000000ull;
__device__ __forceinline__ bool key_is_valid(uint64_t key) {
  return (key >> 24) != 0xFFFFFFFFFFull;
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

constexpr int kMaxRounds = kDispatchChunk / 256;  // 256-assignment rounds per block chunk

// Expert ids of rounds 0 .. rounds-1 of the chunk at `base`, one per thread and round, all
// loads issued before the first is used; ids past N read as 0 (the callers test i < N).
__device__ __forceinline__ void load_chunk_ids(const int32_t* __restrict__ ids, int64_t N,
                                               int64_t base, int rounds,
                                               int (&ev)[kMaxRounds]) {
  const int64_t n = N - base < (int64_t)rounds * 256 ? N - base : (int64_t)rounds * 256;
  const __amdgpu_buffer_rsrc_t r = buffer_rsrc(ids + base, (uint32_t)(n * 4));
#pragma unroll
  for (int q = 0; q < kMaxRounds; ++q)
    ev[q] = (int)__builtin_amdgcn_raw_buffer_load_b32(
        r, q < rounds ? (uint32_t)((q * 256 + (int)threadIdx.x) * 4) : kBufferOOR, 0, 0);
}

// Sum over blocks b < nb of blk_hist[b][e] (total) and over b < before (prefix), with the
// loads issued eight at a time (blocks past nb read as 0).
__device__ __forceinline__ void hist_sums(const int32_t* __restrict__ blk_hist, int nb, int E,
                                          int e, int before, int& tot, int& pre) {
  const __amdgpu_buffer_rsrc_t r = buffer_rsrc(blk_hist, (uint32_t)(nb * (E + 1) * 4));
  tot = 0;
  pre = 0;
  for (int b0 = 0; b0 < nb; b0 += 8) {
    int h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      h[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(
          r, (uint32_t)(((b0 + j) * (E + 1) + e) * 4), 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (b0 + j < before) pre += h[j];
      tot += h[j];
    }
  }
}

}  // namespace

__global__ __launch_bounds__(256) void k_dispatch_hist(const int32_t* __restrict__ ids, int64_t N,
                                                       int E, int chunk,
                                                       int32_t* __restrict__ blk_hist) {
  __shared__ int cnt[260];
  for (int i = threadIdx.x; i <= E; i += 256) cnt[i] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * chunk;
  const int rounds = chunk / 256;
  int ev[kMaxRounds];
  load_chunk_ids(ids, N, base, rounds, ev);
#pragma unroll
  for (int r = 0; r < kMaxRounds; ++r) {
    if (r >= rounds) break;  // uniform
    const int64_t i = base + r * 256 + threadIdx.x;
    const bool valid = i < N;
    int e = valid ? ev[r] : 0;
    if (e < 0 || e >= E) e = E;  // out-of-range ids go to an overflow bucket
    const uint64_t peers = match_key(e, valid);
    if (valid && (peers & lanemask_lt()) == 0) atomicAdd(&cnt[e], __popcll(peers));
  }
  __syncthreads();
  for (int i = threadIdx.x; i <= E; i += 256) blk_hist[(int64_t)blockIdx.x * (E + 1) + i] = cnt[i];
}

__global__ __launch_bounds__(256) void k_dispatch_scatter(
    const int32_t* __restrict__ ids, const float* __restrict__ gates, int64_t N, int E, int cap,
    int nb, int chunk, const int32_t* __restrict__ blk_hist, uint64_t* __restrict__ keys,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ seg_start,
    int32_t* __restrict__ rank, int32_t* __restrict__ slot_of, uint8_t* __restrict__ drop) {
  __shared__ int s_cnt[260], s_run[260], s_kept[260];
  __shared__ int wcnt[4][260];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t base = (int64_t)blockIdx.x * chunk;
  const int rounds = chunk / 256;
  int ev[kMaxRounds];
  float gv[kMaxRounds];
  load_chunk_ids(ids, N, base, rounds, ev);
  {
    const int64_t n = N - base < (int64_t)chunk ? N - base : (int64_t)chunk;
    const __amdgpu_buffer_rsrc_t gr = buffer_rsrc(gates + base, (uint32_t)(n * 4));
#pragma unroll
    for (int q = 0; q < kMaxRounds; ++q)
      gv[q] = buffer_load_f32(gr, q < rounds ? (uint32_t)((q * 256 + tid) * 4) : kBufferOOR);
  }
  for (int e = tid; e <= E; e += 256) {
    int tot, pre;
    hist_sums(blk_hist, nb, E, e, (int)blockIdx.x, tot, pre);
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

#pragma unroll
  for (int r = 0; r < kMaxRounds; ++r) {
    if (r >= rounds || base + r * 256 >= N) break;  // block-uniform
    const int64_t i = base + r * 256 + tid;
    const bool valid = i < N;
    int e = valid ? ev[r] : 0;
    if (e < 0 || e >= E) e = E;
    const uint64_t peers = match_key(e, valid);
    const int wrank = __popcll(peers & lanemask_lt());
    if (valid && wrank == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = s_run[e] + wrank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      rank[pos] = 0;
      if (e < E) {
        keys[pos] = sort_key(gv[r], (uint32_t)i);
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

constexpr int kTile = 256;        // keys per sorted tile (one per thread)
constexpr int kTilesPerItem = 4;  // other tiles one rank work item searches

__device__ __forceinline__ int tiles_of(int n) { return (n + kTile - 1) / kTile; }

// s_pre[e] = exclusive prefix over experts of f(counts[e]), s_pre[E] = total; every thread calls.
template <typename F>
__device__ void expert_prefix(const int32_t* __restrict__ counts, int E, int* s_pre, F f) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) s_pre[e] = e < E ? f(counts[e]) : 0;
  __syncthreads();
  if ((threadIdx.x >> 6) == 0) wave_exclusive_scan(s_pre, E + 1, nullptr);
  __syncthreads();
}

// Bitonic sort of n keys (n a power of two, at most NMAX and the workgroup size), one per
// thread: returns the key that lands at this thread's index in ascending order within its
// aligned group of n threads.  Partners closer than 64 are in the same wave (xor_partner),
// farther ones trade keys through `sk` (one key per thread of LDS).  The network is unrolled
// for NMAX keys and stops after the stage of size n.
template <int NMAX>
__device__ __forceinline__ uint64_t block_bitonic_sort(uint64_t v, uint64_t* sk, int n) {
  const int t = threadIdx.x;
#pragma unroll
  for (int size = 2; size <= NMAX; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (size > n) continue;  // workgroup-uniform
      uint64_t other;
      if (stride >= 64) {
        sk[t] = v;
        __syncthreads();
        other = sk[t ^ stride];
        __syncthreads();
      } else {
        other = xor_partner(v, stride);
      }
      const bool up = (t & size) == 0, lower = (t & stride) == 0;
      // keep the smaller key at the lower index of an ascending pair, the larger otherwise
      v = (lower == up) ? (v < other ? v : other) : (v < other ? other : v);
    }
  }
  return v;
}

// the e with s_pre[e] <= w < s_pre[e+1] (s_pre non-decreasing, w < s_pre[E])
__device__ __forceinline__ int find_expert(const int* s_pre, int E, int w) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= w) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace

__global__ __launch_bounds__(kTile) void k_dispatch_tilesort(uint64_t* __restrict__ keys,
                                                             const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ seg_start,
                                                             int E) {
  __shared__ int s_pre[260];
  __shared__ uint64_t sk[kTile];
  expert_prefix(counts, E, s_pre, [](int n) { return tiles_of(n); });
  const int w = blockIdx.x;
  if (w >= s_pre[E]) return;  // uniform
  const int e = find_expert(s_pre, E, w);
  const int a = w - s_pre[e];
  const int n = counts[e];
  const int m = min(kTile, n - a * kTile);
  const int64_t base = (int64_t)seg_start[e] + (int64_t)a * kTile;
  const int t = threadIdx.x;
  uint64_t v = t < m ? keys[base + t] : ~0ull;  // padding sorts last
  v = block_bitonic_sort<kTile>(v, sk, kTile);
  if (t < m) keys[base + t] = v;
}

// 8 bytes at byte offset `off` of a buffer resource (zeros past its range)
__device__ __forceinline__ uint64_t buffer_load_u64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  return ((uint64_t)v[1] << 32) | v[0];
}

__global__ __launch_bounds__(kTile) void k_dispatch_rank(const uint64_t* __restrict__ keys,
                                                         const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ seg_start,
                                                         int E, int32_t* __restrict__ rank) {
  __shared__ int s_pre[260];
  __shared__ uint64_t sk[kTilesPerItem * kTile];  // the item's group of sorted tiles
  // work items of expert e: (own tile a, group g of kTilesPerItem tiles)
  expert_prefix(counts, E, s_pre, [](int n) {
    const int nt = tiles_of(n);
    return nt * ((nt + kTilesPerItem - 1) / kTilesPerItem);
  });
  const int total = s_pre[E];
  const int t = threadIdx.x;
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int e = find_expert(s_pre, E, w);
    const int n = counts[e];
    const int nt = tiles_of(n);
    const int ng = (nt + kTilesPerItem - 1) / kTilesPerItem;
    const int a = (w - s_pre[e]) / ng, g = (w - s_pre[e]) % ng;
    const int64_t seg = seg_start[e];
    const int own_pos = a * kTile + t;
    const uint64_t mine = own_pos < n ? keys[seg + own_pos] : ~0ull;
    int cnt = 0;
    const int b0 = g * kTilesPerItem, b_end = min(nt, b0 + kTilesPerItem);
    // all tiles of the group in one round trip: branch-free loads (a tile's resource covers
    // only its keys; past them, and past the group, reads zeros the searches never reach)
    uint64_t kv[kTilesPerItem];
#pragma unroll
    for (int bb = 0; bb < kTilesPerItem; ++bb) {
      const int b = b0 + bb;
      const int mb = b < b_end ? min(kTile, n - b * kTile) : 0;
      const __amdgpu_buffer_rsrc_t tile =
          buffer_rsrc(keys + seg + (int64_t)(b < b_end ? b : b0) * kTile, (uint32_t)mb * 8u);
      kv[bb] = buffer_load_u64(tile, (uint32_t)t * 8u);
    }
    __syncthreads();  // the previous item's searches are done with sk
#pragma unroll
    for (int bb = 0; bb < kTilesPerItem; ++bb) sk[bb * kTile + t] = kv[bb];
    __syncthreads();
    for (int b = b0; b < b_end; ++b) {
      if (b == a) {
        cnt += t;  // sorted own tile: t keys are smaller
        continue;
      }
      const int mb = min(kTile, n - b * kTile);
      const uint64_t* st = sk + (b - b0) * kTile;
      int lo = 0, hi = mb;  // first index with st[idx] >= mine
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (st[mid] < mine) lo = mid + 1; else hi = mid;
      }
      cnt += lo;
    }
    if (own_pos < n && cnt) atomicAdd(&rank[seg + own_pos], cnt);
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_dispatch_emit(const uint64_t* __restrict__ keys,
                                                       const int32_t* __restrict__ rank,
                                                       const int32_t* __restrict__ seg_start,
                                                       const int32_t* __restrict__ offsets, int E,
                                                       int k, int cap, int32_t* __restrict__ slot_of,
                                                       int32_t* __restrict__ row_token,
                                                       uint8_t* __restrict__ drop) {
  __shared__ int s_seg[260];
  for (int e = threadIdx.x; e <= E; e += 256) s_seg[e] = seg_start[e];
  __syncthreads();
  const int pos = blockIdx.x * 256 + threadIdx.x;
  if (pos >= s_seg[E]) return;  // past the valid buckets
  const int e = find_expert(s_seg, E, pos);
  const uint64_t key = keys[pos];
  const uint32_t i = (uint32_t)(key & 0xFFFFFFFFull);
  const int r = rank[pos];
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

// ---------------------------------------------------------------- small batches
// Up to kSmallN assignments: the whole dispatch in one workgroup.  Key of assignment i with
// expert e: (e << 56) | (~ord(gate) << 24) | i (expert_key); ascending order is expert, then the
// fill order of that expert.  Ids outside [0, E) get kInvalidKey | i, after every valid key.
// The keys are unique, so the bitonic sort in LDS has one result, the same order the bucketed
// multi-kernel path produces; the rank of a key in its expert is its sorted position minus the
// expert's first position.
constexpr int kSmallN = 1024;  // one key per thread of a 1024-thread workgroup

__global__ __launch_bounds__(1024) void k_dispatch_small(
    const int32_t* __restrict__ ids, const float* __restrict__ gates, int N, int E, int k,
    int cap, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_of, int32_t* __restrict__ row_token, uint8_t* __restrict__ drop) {
  __shared__ uint64_t sk[kSmallN];
  __shared__ int cnt[260], start[260], koff[260];
  const int tid = threadIdx.x;
  int P = 1;
  while (P < N) P <<= 1;
  for (int e = tid; e <= E; e += 1024) cnt[e] = 0;
  __syncthreads();
  uint64_t v = ~0ull;  // this thread's key; padding past N sorts last
  if (tid < N) {
    const int e = ids[tid];
    if (e >= 0 && e < E) {
      v = expert_key(e, gates[tid], (uint32_t)tid);
      atomicAdd(&cnt[e], 1);
    } else {
      v = kInvalidKey | (uint64_t)tid;
    }
  }
  // bitonic sort over threads 0 .. P-1 (threads past P only meet each other)
  v = block_bitonic_sort<kSmallN>(v, sk, P);
  sk[tid] = v;
  __syncthreads();
  // expert starts in sorted order and kept-slot offsets
  for (int e = tid; e <= E; e += 1024) {
    start[e] = e < E ? cnt[e] : 0;
    koff[e] = e < E ? min(cnt[e], cap) : 0;
  }
  __syncthreads();
  if (tid < 64) {
    wave_exclusive_scan(start, E + 1, nullptr);
    wave_exclusive_scan(koff, E + 1, nullptr);
  }
  __syncthreads();
  for (int e = tid; e <= E; e += 1024) {
    if (e < E) counts[e] = cnt[e];
    offsets[e] = koff[e];
  }
  for (int p = tid; p < N; p += 1024) {
    const uint64_t key = sk[p];
    const int i = (int)(key & 0xFFFFFFull);
    const int e = (int)(key >> 56);
    const bool valid = key_is_valid(key);
    const int r = p - start[e];
    if (valid && r < cap) {
      const int slot = koff[e] + r;
      slot_of[i] = slot;
      drop[i] = 0;
      row_token[slot] = i / k;
    } else {
      slot_of[i] = -1;
      drop[i] = 1;
    }
  }
}

// ---------------------------------------------------------------- mid-sized batches
// kSmallN < N <= kMidN assignments: two launches.  The assignments are cut into runs of kRun
// consecutive ones.  k_dispatch_runs sorts each run by the same (expert, fill order) keys as the
// one-workgroup path and records where each expert's keys begin in the sorted run.
// k_dispatch_merge: every workgroup loads all sorted runs into LDS and ranks kMergeKeys of the
// keys.  The rank of a key within its expert is its position in its own run's segment of that
// expert plus, for every other run, the number of that run's keys of the same expert that are
// smaller: branch-free binary searches, four runs side by side so that four LDS reads are in
// flight, kSplit threads per key that each take every kSplit-th run.  The searches are bound by LDS
// throughput, hence few keys per workgroup and many workgroups.  The keys are unique, so these
// ranks are the fill-order positions the other paths compute, and the kernel emits the slots
// straight from them.
constexpr int kRun = 512;
constexpr int kMidN = 16384;
constexpr int kMidRuns = kMidN / kRun;
constexpr int kMergeKeys = 128;  // keys ranked per merge workgroup
constexpr int kSplit = 4;        // threads per key
constexpr int kMergeThreads = kSplit * kMergeKeys;
// k_dispatch_merge's dynamic LDS: every key (a multiple of 2 * kMergeThreads of them, as the
// keys arrive in pairs), then each run's expert starts as 16-bit values (room for the most runs
// and experts, so that every thread stores its share without a guard)
constexpr int merge_key_slots(int n) {
  return (n + 2 * kMergeThreads - 1) / (2 * kMergeThreads) * (2 * kMergeThreads);
}
constexpr int kOffRounds = (kMidRuns * 257 + kMergeThreads - 1) / kMergeThreads;
constexpr size_t merge_lds_bytes(int n) {
  return (size_t)merge_key_slots(n) * 8 + (size_t)kOffRounds * kMergeThreads * 2;
}

__global__ __launch_bounds__(kRun) void k_dispatch_runs(const int32_t* __restrict__ ids,
                                                        const float* __restrict__ gates, int N,
                                                        int E, uint64_t* __restrict__ keys,
                                                        int32_t* __restrict__ run_off,
                                                        int32_t* __restrict__ slot_of,
                                                        uint8_t* __restrict__ drop) {
  __shared__ uint64_t sk[kRun];
  __shared__ int sex[kRun];
  const int t = threadIdx.x;
  const int base = blockIdx.x * kRun, i = base + t;
  const uint32_t n_bytes = (uint32_t)min(kRun, N - base) * 4u;  // both loads issued at once
  const int e = (int)__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(ids + base, n_bytes),
                                                          t * 4, 0, 0);
  const float g = buffer_load_f32(buffer_rsrc(gates + base, n_bytes), (uint32_t)t * 4u);
  uint64_t v = ~0ull;  // padding past N sorts last
  if (i < N) {
    if (e >= 0 && e < E) {
      v = expert_key(e, g, (uint32_t)i);
    } else {  // out-of-range id: dropped here, never ranked
      v = kInvalidKey | (uint64_t)i;
      slot_of[i] = -1;
      drop[i] = 1;
    }
  }
  v = block_bitonic_sort<kRun>(v, sk, kRun);
  if (i < N) keys[i] = v;  // sorted position t of this run
  // run_off[run][e] = keys of experts below e in the run (e = 0 .. E; invalid keys and padding
  // count as expert E): the thread holding the first key of a larger expert writes the starts
  // of every expert it passes
  const int ex = key_is_valid(v) ? (int)(v >> 56) : E;
  sex[t] = ex;
  __syncthreads();
  int32_t* off = run_off + (int64_t)blockIdx.x * (E + 1);
  const int prev = t ? sex[t - 1] : -1;
  for (int e2 = prev + 1; e2 <= ex; ++e2) off[e2] = t;
  if (t == kRun - 1)
    for (int e2 = ex + 1; e2 <= E; ++e2) off[e2] = kRun;
}

__global__ __launch_bounds__(kMergeThreads) void k_dispatch_merge(
    const uint64_t* __restrict__ keys, const int32_t* __restrict__ run_off, int N, int nb, int E,
    int k, int cap, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_of, int32_t* __restrict__ row_token, uint8_t* __restrict__ drop) {
  extern __shared__ uint64_t s_keys[];  // merge_lds_bytes(N)
  __shared__ int s_tot[258], s_koff[258], s_part[kSplit - 1][kMergeKeys];
  const int t = threadIdx.x, E1 = E + 1;
  uint16_t* s_off = reinterpret_cast<uint16_t*>(s_keys + merge_key_slots(N));
  // Every load in flight at once, the expert starts first: the totals below need only them and
  // run while the keys arrive.  Keys come in pairs as 16-byte loads.  With N odd the last
  // pair's second key is the workspace word after the keys (the keys' slice ends on a 256-byte
  // boundary); it and the zeros past it are never searched.
  const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(run_off, (uint32_t)(nb * E1) * 4u);
  int ov[kOffRounds];  // zeros past the nb * E1 starts
#pragma unroll
  for (int q = 0; q < kOffRounds; ++q)
    ov[q] = (int)__builtin_amdgcn_raw_buffer_load_b32(
        ro, (uint32_t)((q * kMergeThreads + t) * 4), 0, 0);
  constexpr int kKeyRounds = kMidN / (2 * kMergeThreads);
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(keys, (uint32_t)((N + 1) / 2) * 16u);
  const int rounds = (N + 2 * kMergeThreads - 1) / (2 * kMergeThreads);
  uint4 kv[kKeyRounds];
#pragma unroll
  for (int q = 0; q < kKeyRounds; ++q)
    kv[q] = buffer_load16(
        rk, q < rounds ? (uint32_t)((q * kMergeThreads + t) * 16) : kBufferOOR);
#pragma unroll
  for (int q = 0; q < kOffRounds; ++q) s_off[q * kMergeThreads + t] = (uint16_t)ov[q];
  __syncthreads();
  // s_tot[e] = valid keys of the experts below e over all runs
  for (int e = t; e <= E; e += kMergeThreads) {
    int sum = 0;
    for (int b = 0; b < nb; ++b) sum += s_off[b * E1 + e];
    s_tot[e] = sum;
  }
  __syncthreads();
  for (int e = t; e <= E; e += kMergeThreads)
    s_koff[e] = e < E ? min(s_tot[e + 1] - s_tot[e], cap) : 0;
  __syncthreads();
  if (t < 64) wave_exclusive_scan(s_koff, E1, nullptr);  // kept-slot offsets
  uint4* s_pairs = reinterpret_cast<uint4*>(s_keys);
#pragma unroll
  for (int q = 0; q < kKeyRounds; ++q)
    if (q < rounds) s_pairs[q * kMergeThreads + t] = kv[q];
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = t; e <= E; e += kMergeThreads) {
      if (e < E) counts[e] = s_tot[e + 1] - s_tot[e];
      offsets[e] = s_koff[e];
    }
  // key p: thread `share` of its kSplit counts the runs b = share, share + kSplit, ...; share 0
  // also counts the key's own position in its own run
  const int tk = t % kMergeKeys, share = t / kMergeKeys;
  const int p = blockIdx.x * kMergeKeys + tk;
  const uint64_t key = s_keys[p < N ? p : 0];
  const bool act = p < N && key_is_valid(key);  // out-of-range ids: dropped by k_dispatch_runs
  const int e = act ? (int)(key >> 56) : 0, run = p / kRun;
  int part = act && share == 0 ? p % kRun - s_off[run * E1 + e] : 0;
  constexpr int G = 4;  // runs searched side by side
  for (int b0 = share; act && b0 < nb; b0 += kSplit * G) {
    int lo[G], len[G], from[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {  // reads of runs past nb land on run 0 and are discarded
      const int b = b0 + kSplit * j;
      const bool other = b < nb && b != run;
      const int bo = (b < nb ? b : 0) * E1 + e;
      const int a = s_off[bo], z = s_off[bo + 1];
      lo[j] = from[j] = other ? b * kRun + a : 0;
      len[j] = other ? z - a : 0;
    }
    // lower bound: lo[j] ends at the first key of run b's segment that is not below `key`.
    // Branch-free steps, so that the G reads of a step are in flight together; a finished
    // search (len 0) reads key 0 and keeps its state.
    int any = 0;
#pragma unroll
    for (int j = 0; j < G; ++j) any |= len[j];
    while (any > 0) {
      uint64_t sv[G];
#pragma unroll
      for (int j = 0; j < G; ++j) sv[j] = s_keys[len[j] > 0 ? lo[j] + (len[j] >> 1) : 0];
      any = 0;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int h = len[j] >> 1;
        const bool below = len[j] > 0 && sv[j] < key;
        lo[j] = below ? lo[j] + h + 1 : lo[j];
        len[j] = below ? len[j] - h - 1 : h;
        any |= len[j];
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) part += lo[j] - from[j];
  }
  if (share > 0) s_part[share - 1][tk] = part;
  __syncthreads();
  if (share > 0 || !act) return;
  int rank = part;
#pragma unroll
  for (int j = 0; j < kSplit - 1; ++j) rank += s_part[j][tk];
  const int i = (int)(key & 0xFFFFFFull);
  if (rank < cap) {
    const int slot = s_koff[e] + rank;
    slot_of[i] = slot;
    drop[i] = 0;
    row_token[slot] = i / k;
  } else {
    slot_of[i] = -1;
    drop[i] = 1;
  }
}

int64_t dispatch_runs(int64_t n) { return n > kSmallN && n <= kMidN ? (n + kRun - 1) / kRun : 0; }

// ---------------------------------------------------------------- routed token rows
// x_routed[s] = x[row_token[s]] for every kept slot s < offsets[E]: the token rows copied into
// expert-slot order, the rows the first expert GEMM reads (fused-MoE flow diagram, GEMM 1 box:
// the reorder happens on the way into the expert GEMMs).  HBM-bound copy: one wave per slot
// row, 16-byte chunks (row_bytes a multiple of 16 and both bases 16-byte aligned) or 4-byte
// words, every load of a batch issued before its stores.  The grid covers an upper bound on the
// kept rows; waves past offsets[E] return.
__global__ __launch_bounds__(256) void k_gather_rows(const char* __restrict__ x,
                                                     const int32_t* __restrict__ row_token,
                                                     const int32_t* __restrict__ offsets, int E,
                                                     int row_bytes, bool vec16,
                                                     char* __restrict__ out) {
  constexpr int kB = 4;
  const int lane = threadIdx.x & 63;
  const int64_t s = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (s >= offsets[E]) return;
  const int64_t t = row_token[s];
  const char* src = x + t * row_bytes;
  char* dst = out + s * row_bytes;
  if (vec16) {
    const int nch = row_bytes / 16;
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(src, (uint32_t)row_bytes);
    for (int c0 = lane; c0 < nch; c0 += 64 * kB) {
      uint4 v[kB];
#pragma unroll
      for (int b = 0; b < kB; ++b) v[b] = buffer_load16(r, (uint32_t)(c0 + 64 * b) * 16u);
#pragma unroll
      for (int b = 0; b < kB; ++b)
        if (c0 + 64 * b < nch) reinterpret_cast<uint4*>(dst)[c0 + 64 * b] = v[b];
    }
  } else {
    const int nw = row_bytes / 4;
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(src, (uint32_t)row_bytes);
    for (int c0 = lane; c0 < nw; c0 += 64 * kB) {
      uint32_t v[kB];
#pragma unroll
      for (int b = 0; b < kB; ++b)
        v[b] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)((c0 + 64 * b) * 4), 0, 0);
#pragma unroll
      for (int b = 0; b < kB; ++b)
        if (c0 + 64 * b < nw) reinterpret_cast<uint32_t*>(dst)[c0 + 64 * b] = v[b];
    }
  }
}

hipError_t launch_gather_rows(const moe_shape& s, const void* x, const int32_t* row_token,
                              const int32_t* offsets, void* x_routed, hipStream_t st) {
  const int64_t rows_ub = max_rows(s);
  if (rows_ub <= 0) return hipSuccess;
  const int row_bytes = s.d_model * (s.dtype == MOE_BF16 ? 2 : 4);
  const bool vec16 = row_bytes % 16 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)x_routed % 16 == 0;
  hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)((rows_ub + 3) / 4)), dim3(256), 0, st,
                     (const char*)x, row_token, offsets, s.n_experts, row_bytes, vec16,
                     (char*)x_routed);
  return hipGetLastError();
}

// ---------------------------------------------------------------- padded fixed buffers
// "Some Tokens Do Not Get In", "Why there is a buffer": each expert owns a buffer of `cap`
// slots whether or not it fills them, and the unused slots are computed anyway.  From the
// compact result: the kept assignment of rank r of expert e moves to slot e * cap + r, buffer
// row e * cap + r takes the token of that assignment or -1 (a zero row) when r is past the
// expert's kept count, and the padded offsets are e * cap.  Thread id covers assignment id and
// buffer row id.
__global__ __launch_bounds__(256) void k_pad_layout(const int32_t* __restrict__ ids,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ row_token,
                                                    int64_t N, int E, int cap,
                                                    int32_t* __restrict__ slot_of,
                                                    int32_t* __restrict__ row_token_pad,
                                                    int32_t* __restrict__ offsets_pad) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id < N) {
    const int sl = slot_of[id];
    if (sl >= 0) {
      const int e = ids[id];  // kept => 0 <= e < E
      slot_of[id] = e * cap + (sl - offsets[e]);
    }
  }
  if (id < (int64_t)E * cap) {
    const int e = (int)(id / cap), r = (int)(id % cap);
    const int kept = offsets[e + 1] - offsets[e];
    row_token_pad[id] = r < kept ? row_token[offsets[e] + r] : -1;
  }
  if (id <= E) offsets_pad[id] = (int)id * cap;
}

hipError_t launch_pad_layout(const moe_shape& s, const int32_t* ids, const int32_t* offsets,
                             const int32_t* row_token, int32_t* slot_of, int32_t* row_token_pad,
                             int32_t* offsets_pad, hipStream_t st) {
  const int64_t N = s.T * (int64_t)s.top_k;
  const int64_t rows = (int64_t)s.n_experts * s.capacity;
  int64_t n = N > rows ? N : rows;
  if (n < s.n_experts + 1) n = s.n_experts + 1;
  hipLaunchKernelGGL(k_pad_layout, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ids,
                     offsets, row_token, N, s.n_experts, s.capacity, slot_of, row_token_pad,
                     offsets_pad);
  return hipGetLastError();
}

// ---------------------------------------------------------------- dropless pair grouping
// Fused-MoE flow diagram (moe-vllm flow), note on the GEMM boxes: both GEMMs walk the pairs
// sorted by expert so that every block uses one expert's weights; nothing is dropped.  Pair
// p = t * k + c goes to position offsets[e] + #{q < p : ids[q] = e} (a stable counting sort
// by expert id), with row_token = p / k beside it.  Pairs with ids outside [0, E) land after
// offsets[E], where no GEMM tile reads.  Same wave-ballot ranking as k_dispatch_scatter; with
// a single block (N <= chunk) the block counts its own chunk, so no histogram kernel runs
// before it.
__global__ __launch_bounds__(256) void k_dispatch_pairs(
    const int32_t* __restrict__ ids, int64_t N, int E, int k, int nb, int chunk,
    const int32_t* __restrict__ blk_hist, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ row_token) {
  __shared__ int s_cnt[260], s_run[260];
  __shared__ int wcnt[4][260];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t base = (int64_t)blockIdx.x * chunk;
  const int rounds = chunk / 256;
  int ev[kMaxRounds];
  load_chunk_ids(ids, N, base, rounds, ev);
  for (int e = tid; e <= E; e += 256) {
    s_cnt[e] = 0;
    s_run[e] = 0;
    for (int w = 0; w < 4; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();
  if (blk_hist) {  // totals and the prefix of the blocks before this one
    for (int e = tid; e <= E; e += 256) {
      int tot, pre;
      hist_sums(blk_hist, nb, E, e, (int)blockIdx.x, tot, pre);
      s_cnt[e] = tot;
      s_run[e] = pre;
    }
  } else {  // the only block: count its own chunk
#pragma unroll
    for (int r = 0; r < kMaxRounds; ++r) {
      if (r >= rounds) break;  // uniform
      const int64_t i = base + r * 256 + tid;
      const bool valid = i < N;
      int e = valid ? ev[r] : 0;
      if (e < 0 || e >= E) e = E;
      const uint64_t peers = match_key(e, valid);
      if (valid && (peers & lanemask_lt()) == 0) atomicAdd(&s_cnt[e], __popcll(peers));
    }
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = tid; e < E; e += 256) counts[e] = s_cnt[e];
  __syncthreads();
  if (wave == 0) wave_exclusive_scan(s_cnt, E + 1, nullptr);  // bucket starts; [E] = valid pairs
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = tid; e <= E; e += 256) offsets[e] = s_cnt[e];
  for (int e = tid; e <= E; e += 256) s_run[e] += s_cnt[e];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kMaxRounds; ++r) {
    if (r >= rounds || base + r * 256 >= N) break;  // block-uniform
    const int64_t i = base + r * 256 + tid;
    const bool valid = i < N;
    int e = valid ? ev[r] : 0;
    if (e < 0 || e >= E) e = E;
    const uint64_t peers = match_key(e, valid);
    const int wrank = __popcll(peers & lanemask_lt());
    if (valid && wrank == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = s_run[e] + wrank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      sorted_pairs[pos] = (int32_t)i;
      row_token[pos] = (int32_t)(i / k);
    }
    __syncthreads();
    for (int ee = tid; ee <= E; ee += 256) {
      s_run[ee] += wcnt[0][ee] + wcnt[1][ee] + wcnt[2][ee] + wcnt[3][ee];
      wcnt[0][ee] = wcnt[1][ee] = wcnt[2][ee] = wcnt[3][ee] = 0;
    }
    __syncthreads();
  }
}

int dispatch_chunk(int64_t n, bool pairs) {
  if (pairs && n <= kDispatchChunk) return kDispatchChunk;  // one block, no histogram launch
  // about 32 blocks: every block sums the histograms of the blocks before it, so many more
  // blocks cost more in those sums than their extra parallelism saves
  int64_t c = (n / 32 + 255) / 256 * 256;
  if (c < 256) c = 256;
  if (c > kDispatchChunk) c = kDispatchChunk;
  return (int)c;
}

int64_t dispatch_blocks(int64_t n, bool pairs) {
  const int c = dispatch_chunk(n, pairs);
  return (n + c - 1) / c;
}

hipError_t launch_dispatch_pairs(const moe_shape& s, const int32_t* ids, int32_t* counts,
                                 int32_t* offsets, int32_t* sorted_pairs, int32_t* row_token,
                                 int32_t* blk_hist, hipStream_t st) {
  const int64_t N = s.T * (int64_t)s.top_k;
  const int E = s.n_experts;
  const int chunk = dispatch_chunk(N, true);
  const int nb = (int)dispatch_blocks(N, true);
  if (nb > 1)
    hipLaunchKernelGGL(k_dispatch_hist, dim3(nb), dim3(256), 0, st, ids, N, E, chunk, blk_hist);
  hipLaunchKernelGGL(k_dispatch_pairs, dim3(nb), dim3(256), 0, st, ids, N, E, s.top_k, nb, chunk,
                     nb > 1 ? (const int32_t*)blk_hist : nullptr, counts, offsets, sorted_pairs,
                     row_token);
  return hipGetLastError();
}

hipError_t launch_dispatch(const moe_shape& s, const int32_t* ids, const float* gates,
                           int32_t* counts, int32_t* offsets, int32_t* slot_of,
                           int32_t* row_token, uint8_t* drop, int32_t* seg_start,
                           int32_t* blk_hist, uint64_t* keys, int32_t* rank, hipStream_t st) {
  const int64_t N = s.T * (int64_t)s.top_k;
  const int E = s.n_experts;
  if (N <= kSmallN) {
    hipLaunchKernelGGL(k_dispatch_small, dim3(1), dim3(1024), 0, st, ids, gates, (int)N, E,
                       s.top_k, s.capacity, counts, offsets, slot_of, row_token, drop);
    return hipGetLastError();
  }
  if (N <= kMidN) {
    static std::atomic<bool> lds_allowed[kMaxDevices];
    if (hipError_t err = allow_dynamic_lds((const void*)k_dispatch_merge,
                                           (int)merge_lds_bytes(kMidN), lds_allowed);
        err != hipSuccess)
      return err;
    const int nb = (int)dispatch_runs(N);
    hipLaunchKernelGGL(k_dispatch_runs, dim3(nb), dim3(kRun), 0, st, ids, gates, (int)N, E, keys,
                       blk_hist, slot_of, drop);
    hipLaunchKernelGGL(k_dispatch_merge, dim3((unsigned)((N + kMergeKeys - 1) / kMergeKeys)),
                       dim3(kMergeThreads), merge_lds_bytes((int)N), st, keys, blk_hist, (int)N,
                       nb, E, s.top_k, s.capacity, counts, offsets, slot_of, row_token, drop);
    return hipGetLastError();
  }
  const int chunk = dispatch_chunk(N);
  const int nb = (int)dispatch_blocks(N);
  hipLaunchKernelGGL(k_dispatch_hist, dim3(nb), dim3(256), 0, st, ids, N, E, chunk, blk_hist);
  hipLaunchKernelGGL(k_dispatch_scatter, dim3(nb), dim3(256), 0, st, ids, gates, N, E, s.capacity,
                     nb, chunk, blk_hist, keys, counts, offsets, seg_start, rank, slot_of, drop);
  const int tiles_ub = (int)((N + kTile - 1) / kTile) + E;  // >= sum over experts of tiles
  hipLaunchKernelGGL(k_dispatch_tilesort, dim3(tiles_ub), dim3(kTile), 0, st, keys, counts,
                     seg_start, E);
  hipLaunchKernelGGL(k_dispatch_rank, dim3(1024), dim3(kTile), 0, st, keys, counts, seg_start, E,
                     rank);
  hipLaunchKernelGGL(k_dispatch_emit, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, keys,
                     rank, seg_start, offsets, E, s.top_k, s.capacity, slot_of, row_token, drop);
  return hipGetLastError();
}

}  // namespace moe
