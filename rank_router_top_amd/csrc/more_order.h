// more_order.h -- expert sweep order for a biased router, and per-call
// statistics of the packed weights.
//
// The order (experts by bias descending, ties by index ascending) is a speed
// choice only: high-bias experts tend to end in the top-k, so sweeping them
// first lets a short seed pass bound the k-th logit closely.  The selected set
// and its output order never depend on it.  Expert j's position is the number
// of experts that precede it, counted over all pairs in parallel: M / 16
// workgroups of 16 experts x 16 slices, the bias staged in LDS (M <= 16384,
// O(M^2 / 65536) compares per thread).  Larger biased routers keep the index
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

__global__ __launch_bounds__(256) void order_count_kernel(OrderArgs a) {
  __shared__ float bs[kOrderMaxM];
  __shared__ int part[16][16];
  for (int i = threadIdx.x; i < a.M; i += 256) bs[i] = a.bias[i];
  __syncthreads();
  const int jj = threadIdx.x & 15, sl = threadIdx.x >> 4;
  const int j = blockIdx.x * 16 + jj;
  int cnt = 0;
  if (j < a.M) {
    const float bj = bs[j];
    // slice sl counts experts i = sl, sl + 16, ... ahead of j: larger bias,
    // or equal bias and lower index
    for (int i = sl; i < a.M; i += 16) {
      const float bi = bs[i];
      cnt += (bi > bj || (bi == bj && i < j)) ? 1 : 0;
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

// Per-call statistics of the packed weights, for the routing kernel's error
// bound and seed pass (one workgroup):
//   bmin[t]   smallest bias of sweep tile t's experts (0 without a bias), or
//             -inf when the tile holds padding positions;
//   wstat[0]  max over experts of the column norm ||R2[:, m]||_2;
//   wstat[1]  max over experts of |b_m| (0 without a bias);
//   wstat[2]  (int bits) seed-pass length of the sweep: seed_tiles when the
//             experts are in bias-descending order, every tile otherwise;
//   status    the routing calls' stall word, cleared.
struct TileStatArgs {
  const float* bias;      // M or null
  const int* perm;        // [Mpad] position -> expert (-1 on padding)
  const float* colnorm2;  // [Mpad] squared column norm per position (0 on padding)
  int Mpad, NT;
  int ordered;            // 1: perm is the bias-descending order
  int seed_tiles;         // seed length for the ordered case (<= NT)
  float* bmin;
  float* wstat;
  int* status;
};

__global__ __launch_bounds__(1024) void tilestat_kernel(TileStatArgs a) {
  __shared__ float red[2][16];
  float nmax = 0.f, babs = 0.f;
  for (int p = threadIdx.x; p < a.Mpad; p += 1024) {
    nmax = fmaxf(nmax, a.colnorm2[p]);
    const int j = a.perm[p];
    if (a.bias && j >= 0) babs = fmaxf(babs, fabsf(a.bias[j]));
  }
  for (int t = threadIdx.x; t < a.NT; t += 1024) {
    float mn = __builtin_inff();
    bool pad = false;
    for (int i = 0; i < 32; ++i) {
      const int j = a.perm[t * 32 + i];
      if (j < 0) pad = true;
      else mn = fminf(mn, a.bias ? a.bias[j] : 0.f);
    }
    a.bmin[t] = pad ? -__builtin_inff() : mn;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    nmax = fmaxf(nmax, __shfl_xor(nmax, o));
    babs = fmaxf(babs, __shfl_xor(babs, o));
  }
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wv] = nmax;
    red[1][wv] = babs;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float n = 0.f, b = 0.f;
    for (int q = 0; q < 16; ++q) {
      n = fmaxf(n, red[0][q]);
      b = fmaxf(b, red[1][q]);
    }
    a.wstat[0] = __builtin_sqrtf(n);
    a.wstat[1] = b;
    a.wstat[2] = __int_as_float(a.ordered ? a.seed_tiles : a.NT);
    *a.status = 0;
  }
}

}  // namespace more
