// Batch consolidation: the Token Scheduler of "Token Routing Optimization in Batch Processing".
//
// The diagram keeps every token's routing and changes only which tokens travel together: two
// batches that each activate every expert with one token per expert become two batches that
// each activate half the experts with two tokens per expert.  For a decode-sized batch the
// expert GEMMs stream the weights of every active expert once, so fewer active experts per
// batch means fewer weight bytes per batch.
//
// Order used (the pages give none): tokens sorted by their expert set (the k ids sorted
// ascending, compared as a tuple), ties by token index, then cut into consecutive batches of
// the original size.  The whole pool is sorted by one workgroup: key = the sorted ids packed
// most significant first (bits_e bits each, id E standing for an id outside [0, E)), then the
// token index (13 bits); the keys are unique, so the bitonic network has one result.
//
// Kernels:
//   k_schedule_sort  one 1024-thread workgroup, up to kSchedMaxT keys in LDS;
//   k_batch_experts  one wave per batch: the distinct experts its tokens are routed to, from a
//                    per-wave expert bitmask in LDS;
//   k_permute_rows   one wave per row: row gather (dst[i] = src[idx[i]]) or scatter
//                    (dst[idx[i]] = src[i]) with 16-byte (or 4-byte) accesses.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(1024) void k_schedule_sort(const int32_t* __restrict__ ids, int T,
                                                        int k, int E, int bits_e,
                                                        int32_t* __restrict__ order) {
  __shared__ uint64_t sk[kSchedMaxT];
  const int tid = threadIdx.x;
  int P = 1;
  while (P < T) P <<= 1;
  for (int i = tid; i < P; i += 1024) {
    uint64_t key = ~0ull;  // padding sorts last
    if (i < T) {
      int v[kSchedMaxK];
      for (int c = 0; c < k; ++c) {
        const int e = ids[(int64_t)i * k + c];
        v[c] = (e < 0 || e >= E) ? E : e;
      }
      for (int c = 1; c < k; ++c) {  // insertion sort of the k ids
        const int a = v[c];
        int j = c - 1;
        while (j >= 0 && v[j] > a) {
          v[j + 1] = v[j];
          --j;
        }
        v[j + 1] = a;
      }
      key = 0;
      for (int c = 0; c < k; ++c) key = (key << bits_e) | (uint64_t)v[c];
      key = (key << kSchedIndexBits) | (uint64_t)i;
    }
    sk[i] = key;
  }
  __syncthreads();
  // bitonic network over P keys: pair (lo, lo + j) with bit j of lo clear, ascending where bit
  // `size` of lo is clear
  for (int size = 2; size <= P; size <<= 1) {
    for (int j = size >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P / 2; i += 1024) {
        const int lo = 2 * j * (i / j) + (i % j), hi = lo + j;
        const bool up = (lo & size) == 0;
        const uint64_t a = sk[lo], b = sk[hi];
        if ((a > b) == up) {
          sk[lo] = b;
          sk[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < T; i += 1024)
    order[i] = (int32_t)(sk[i] & ((1ull << kSchedIndexBits) - 1));
}

// Active experts of batch b = the tokens at positions b * B .. b * B + B - 1: token order[i] at
// position i, or token i without an order.
__global__ __launch_bounds__(256) void k_batch_experts(const int32_t* __restrict__ ids,
                                                       const int32_t* __restrict__ order, int B,
                                                       int M, int k, int E,
                                                       int32_t* __restrict__ out) {
  __shared__ uint32_t mask[4][8];  // one 256-bit expert set per wave
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + wave;
  if (lane < 8) mask[wave][lane] = 0u;
  __syncthreads();
  if (b < M) {
    for (int j = lane; j < B * k; j += 64) {
      const int64_t pos = (int64_t)b * B + j / k;
      const int64_t t = order ? (int64_t)order[pos] : pos;
      const int e = ids[t * k + j % k];
      if (e >= 0 && e < E) atomicOr(&mask[wave][e >> 5], 1u << (e & 31));
    }
  }
  __syncthreads();
  if (b < M && lane == 0) {
    int n = 0;
    for (int w = 0; w < 8; ++w) n += __popc(mask[wave][w]);
    out[b] = n;
  }
}

__global__ __launch_bounds__(256) void k_permute_rows(const unsigned char* __restrict__ src,
                                                      const int32_t* __restrict__ idx,
                                                      unsigned char* __restrict__ dst, int64_t n,
                                                      int row_bytes, int scatter) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (i >= n) return;
  const int64_t r = idx[i];
  const unsigned char* s = src + (scatter ? i : r) * row_bytes;
  unsigned char* d = dst + (scatter ? r : i) * row_bytes;
  if (row_bytes % 16 == 0) {
    for (int c = lane; c < row_bytes / 16; c += 64)
      reinterpret_cast<uint4*>(d)[c] = reinterpret_cast<const uint4*>(s)[c];
  } else {
    for (int c = lane; c < row_bytes / 4; c += 64)
      reinterpret_cast<uint32_t*>(d)[c] = reinterpret_cast<const uint32_t*>(s)[c];
  }
}

int schedule_bits_e(int E) {
  int b = 0;
  while ((1 << b) <= E) ++b;  // values 0 .. E
  return b;
}

hipError_t launch_schedule(const int32_t* ids, int T, int k, int E, int32_t* order,
                           hipStream_t st) {
  hipLaunchKernelGGL(k_schedule_sort, dim3(1), dim3(1024), 0, st, ids, T, k, E,
                     schedule_bits_e(E), order);
  return hipGetLastError();
}

hipError_t launch_batch_experts(const int32_t* ids, const int32_t* order, int B, int M, int k,
                                int E, int32_t* out, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_batch_experts, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, st, ids, order,
                     B, M, k, E, out);
  return hipGetLastError();
}

hipError_t launch_permute_rows(const void* src, const int32_t* idx, void* dst, int64_t n,
                               int row_bytes, bool scatter, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_permute_rows, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st,
                     (const unsigned char*)src, idx, (unsigned char*)dst, n, row_bytes,
                     scatter ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
