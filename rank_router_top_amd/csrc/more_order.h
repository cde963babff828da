// more_order.h -- expert sweep order for a biased router.
//
// The order (experts by bias descending, ties by index ascending) is a speed
// choice only: high-bias experts tend to end in the top-k, so sweeping them
// first lets a short seed pass bound the k-th logit closely.  The selected set
// and its output order never depend on it.  Expert j's position is the number
// of experts that precede it, counted over all pairs in parallel: M / 16
// workgroups of 16 experts x 16 contiguous slices, the bias staged in LDS
// in chunks (M <= 16384, M / 16 compares per thread).  Larger biased routers keep the index
// order (and seed over every tile).
#pragma once
#include "more_device.h"

namespace more {

constexpr int kOrderMaxM = 16384;   // largest M that gets the bias-descending order

struct OrderArgs {
  const float* bias;   // M
  int M, Mpad;
  int* perm;           // [Mpad]: position -> expert (-1 on padding)
};

// The bias is staged in LDS 2048 entries (8 KiB) at a time, small enough for
// the workgroups to run beside the projection kernel (the whole routing call
// packs the sweep operands on a side stream while the projection streams X).
constexpr int kOrderChunk = 2048;

__global__ __launch_bounds__(256) void order_count_kernel(OrderArgs a) {
  // a chunk of the bias in LDS, padded with -inf to a multiple of 64 (a
  // padding entry is never ahead of a real expert: it is not larger, and a
  // tie needs i < j < M)
  __shared__ __align__(16) float bs[kOrderChunk];
  __shared__ int part[16][16];
  const int mp = (a.M + 63) & ~63;
  const int jj = threadIdx.x & 15, sl = threadIdx.x >> 4;
  const int j = blockIdx.x * 16 + jj;
  const float bj = j < a.M ? a.bias[j] : 0.f;
  int cnt = 0;
  for (int c0 = 0; c0 < mp; c0 += kOrderChunk) {
    const int cl = mp - c0 < kOrderChunk ? mp - c0 : kOrderChunk;   // a multiple of 64
    __syncthreads();   // the previous chunk has been read
    for (int i = threadIdx.x; i < cl; i += 256) bs[i] = c0 + i < a.M ? a.bias[c0 + i] : -__builtin_inff();
    __syncthreads();
    if (j < a.M) {
      // slice sl of the chunk, read 4 at a time; an expert is ahead of j if
      // its bias is larger, or equal with a lower index
      const int len = cl / 16;   // a multiple of 4
      const int i0 = sl * len;
      const float4* b4 = (const float4*)(bs + i0);
#pragma unroll 4
      for (int q = 0; q < len / 4; ++q) {
        const float4 v = b4[q];
        const int i = c0 + i0 + 4 * q;
        cnt += (v.x > bj || (v.x == bj && i < j)) ? 1 : 0;
        cnt += (v.y > bj || (v.y == bj && i + 1 < j)) ? 1 : 0;
        cnt += (v.z > bj || (v.z == bj && i + 2 < j)) ? 1 : 0;
        cnt += (v.w > bj || (v.w == bj && i + 3 < j)) ? 1 : 0;
      }
    }
  }
  part[sl][jj] = cnt;
  __syncthreads();
  if (sl == 0 && j < a.Mpad) {
    if (j < a.M) {
      int pos = 0;
      for (int q = 0; q < 16; ++q) pos += part[q][jj];
      a.perm[pos] = j;
    } else {
      a.perm[j] = -1;   // padding keeps its own position (after every expert)
    }
  }
}

}  // namespace more
