// more_order.h -- expert sweep order for a biased router.
//
// The order (experts by bias descending, ties by index ascending) is a speed
// choice only: high-bias experts tend to end in the top-k, so sweeping them
// first lets a short seed pass bound the k-th logit closely.  The selected set
// and its output order never depend on it.
//
// Two kernels, O(M log M) work, each with 8 KiB of LDS (small enough to run
// beside the projection kernel: the whole routing call packs the sweep
// operands on a side stream while the projection streams X):
//   order_sort_kernel   one workgroup per chunk of 2048 experts sorts the
//                       chunk's keys (bias mapped to an order-preserving
//                       32-bit integer) descending with a bitonic network
//                       (keys in registers, exchanged by lane shuffles inside
//                       a wave and through LDS across waves) and writes the
//                       sorted chunk to the workspace;
//   order_rank_kernel   expert j's position is the number of experts ahead of
//                       it: in every chunk, a binary search counts the keys
//                       above j's (chunks of lower index count equal keys as
//                       ahead, chunks of higher index do not; inside j's own
//                       chunk equal keys of lower index are counted directly,
//                       only when the chunk holds such a tie).
// M <= 16384 (8 chunks); larger biased routers keep the index order (and seed
// over every tile).
#pragma once
#include "more_device.h"

namespace more {

constexpr int kOrderMaxM = 16384;   // largest M that gets the bias-descending order
constexpr int kOrderChunk = 2048;   // experts per sorted chunk (8 KiB of keys in LDS)
constexpr int kOrderThreads = 256;

struct OrderArgs {
  const float* bias;   // M
  int M, Mpad;
  uint32_t* keys;      // [ceil(M / kOrderChunk) * kOrderChunk]: sorted chunks (workspace)
  int* perm;           // [Mpad]: position -> expert (-1 on padding)
};

// Order-preserving map of a float onto uint32 (a larger float gives a larger
// key; -0 and +0 give the same key).  Every non-NaN float maps above 0, so 0
// pads a chunk past M and is never counted as ahead of a real expert.
__device__ __forceinline__ uint32_t order_key(float b) {
  const uint32_t u = __float_as_uint(b == 0.f ? 0.f : b);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Thread t holds the keys at positions t and t + 1024 of the chunk in
// registers.  A step of the network pairs position i with i ^ stride: for
// strides up to 32 the partner sits in the same wave (a lane shuffle), for
// 64 .. 512 in another wave (exchanged through LDS between two workgroup
// barriers), and 1024 is the thread's other key.
constexpr int kOrderSortThreads = kOrderChunk / 2;

// The key position `pos` keeps after its compare-exchange with partner key y:
// in a descending run the lower position of the pair takes the larger key, in
// an ascending run the smaller.
__device__ __forceinline__ uint32_t order_keep(uint32_t x, uint32_t y, int pos, int size, int stride) {
  const bool desc = (pos & size) == 0, lower = (pos & stride) == 0;
  const uint32_t mx = x > y ? x : y, mn = x > y ? y : x;
  return lower == desc ? mx : mn;
}

__global__ __launch_bounds__(kOrderSortThreads) void order_sort_kernel(OrderArgs a) {
  __shared__ uint32_t s[kOrderChunk];
  const int c0 = blockIdx.x * kOrderChunk;
  const int t = threadIdx.x;
  uint32_t v[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = c0 + t + q * kOrderSortThreads;
    v[q] = i < a.M ? order_key(a.bias[i]) : 0u;
  }
  // bitonic network: runs of `size` are sorted descending where (i & size) is
  // 0 and ascending otherwise, then merged; the last merge (size = chunk)
  // leaves the whole chunk descending
  for (int size = 2; size <= kOrderChunk; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      uint32_t y[2];
      if (stride == kOrderSortThreads) {
        y[0] = v[1];
        y[1] = v[0];
      } else if (stride >= 64) {
        __syncthreads();   // the previous exchange has been read
        s[t] = v[0];
        s[t + kOrderSortThreads] = v[1];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 2; ++q) y[q] = s[(t + q * kOrderSortThreads) ^ stride];
      } else {
#pragma unroll
        for (int q = 0; q < 2; ++q) y[q] = (uint32_t)__shfl_xor((int)v[q], stride);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) v[q] = order_keep(v[q], y[q], t + q * kOrderSortThreads, size, stride);
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) a.keys[c0 + t + q * kOrderSortThreads] = v[q];
}

// Number of keys above x in a descending chunk of kOrderChunk keys.
__device__ __forceinline__ int order_count_above(const uint32_t* s, uint32_t x) {
  int pos = 0;   // s[0 .. pos) > x
#pragma unroll
  for (int step = kOrderChunk / 2; step > 0; step >>= 1)
    if (s[pos + step - 1] > x) pos += step;
  // pos = min(count, chunk - 1): only a full chunk of larger keys is left
  return pos + (s[pos] > x ? 1 : 0);
}

__global__ __launch_bounds__(kOrderThreads) void order_rank_kernel(OrderArgs a) {
  constexpr int kPer = kOrderChunk / kOrderThreads / 4;   // 16-byte loads per thread and chunk
  __shared__ __align__(16) uint32_t s[kOrderChunk];
  const int j = blockIdx.x * kOrderThreads + threadIdx.x;
  const bool real = j < a.M;
  const uint32_t kj = real ? order_key(a.bias[j]) : 0u;   // > 0 for a real expert
  const int cj = j / kOrderChunk;
  const int nch = (a.M + kOrderChunk - 1) / kOrderChunk;
  const uint4* kg = (const uint4*)a.keys;
  uint4 nx[kPer];   // the next chunk, in flight while the current one is searched
#pragma unroll
  for (int q = 0; q < kPer; ++q) nx[q] = kg[q * kOrderThreads + threadIdx.x];
  int pos = 0;
  for (int c = 0; c < nch; ++c) {
    __syncthreads();   // the previous chunk has been searched
#pragma unroll
    for (int q = 0; q < kPer; ++q) ((uint4*)s)[q * kOrderThreads + threadIdx.x] = nx[q];
    __syncthreads();
    if (c + 1 < nch) {
#pragma unroll
      for (int q = 0; q < kPer; ++q) nx[q] = kg[(c + 1) * (kOrderChunk / 4) + q * kOrderThreads + threadIdx.x];
    }
    if (real) {
      const int gt = order_count_above(s, kj);
      if (c < cj) {
        pos += order_count_above(s, kj - 1);   // keys >= kj: lower indices, ahead on a tie
      } else if (c > cj) {
        pos += gt;
      } else {
        pos += gt;
        if (order_count_above(s, kj - 1) - gt > 1) {
          // equal keys in j's own chunk: those of lower index are ahead
          for (int i = c * kOrderChunk; i < j; ++i) pos += order_key(a.bias[i]) == kj ? 1 : 0;
        }
      }
    }
  }
  if (real)
    a.perm[pos] = j;
  else if (j < a.Mpad)
    a.perm[j] = -1;   // padding keeps its own position (after every expert)
}

}  // namespace more
