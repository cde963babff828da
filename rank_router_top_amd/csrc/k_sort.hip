// Expert dispatch sort + count: kernels and launch.
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. E, Fig. 9 (sort + count after the router).
#include "more_sort.h"

namespace more {

__device__ __forceinline__ int sort_digit(int key, int shift) { return (int)(((unsigned)key >> shift) & (kSortBuckets - 1)); }

// Lanes of the wave holding digit d (among the lanes where ok is set).
__device__ __forceinline__ unsigned long long sort_peers(int d, bool ok) {
  unsigned long long peers = __builtin_amdgcn_ballot_w64(ok);
#pragma unroll
  for (int bit = 0; bit < kSortDigitBits; ++bit) {
    const unsigned long long b = __builtin_amdgcn_ballot_w64(((d >> bit) & 1) != 0);
    peers &= ((d >> bit) & 1) ? b : ~b;
  }
  return peers;
}

// Per-block digit counts: all keys of the lane are loaded first (one batch of
// independent loads), then each group of lanes with equal digits adds its
// size once.
__global__ __launch_bounds__(kSortThreads) void sort_hist_kernel(SortPassArgs a) {
  __shared__ int h[kSortBuckets];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  if (threadIdx.x < kSortBuckets) h[threadIdx.x] = 0;
  const long long e0 = (long long)blockIdx.x * kSortBlock + (long long)w * 64 * kSortRounds + lane;
  int key[kSortRounds];
#pragma unroll
  for (int r = 0; r < kSortRounds; ++r) key[r] = e0 + r * 64 < a.n ? a.keys_in[e0 + r * 64] : 0;
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < kSortRounds; ++r) {
    const bool ok = e0 + r * 64 < a.n;
    const int d = sort_digit(key[r], a.shift);
    const unsigned long long peers = sort_peers(d, ok);
    if (ok && (peers & lt) == 0) atomicAdd(&h[d], __builtin_popcountll(peers));
  }
  __syncthreads();
  if (threadIdx.x < kSortBuckets) a.hist[(size_t)threadIdx.x * a.B + blockIdx.x] = h[threadIdx.x];
}

// One workgroup per digit d: in-place exclusive scan of row d of the
// (digit, block) counts, and the row total in tot[d].
__global__ __launch_bounds__(kSortScanThreads) void sort_scan_kernel(int* hist, int* tot, int B) {
  constexpr int kWaves = kSortScanThreads / 64;
  __shared__ int wsum[kWaves];
  __shared__ int carry_s;
  const int d = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry_s = 0;
  int* row = hist + (size_t)d * B;
  for (int c0 = 0; c0 < B; c0 += kSortScanThreads) {
    const int i = c0 + threadIdx.x;
    const int v = i < B ? row[i] : 0;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    __syncthreads();   // wsum and carry_s of the previous chunk have been read
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int before = carry_s;
    for (int k = 0; k < wv; ++k) before += wsum[k];
    if (i < B) row[i] = before + x - v;
    __syncthreads();
    if (threadIdx.x == kSortScanThreads - 1) carry_s = before + x;
  }
  __syncthreads();
  if (threadIdx.x == 0) tot[d] = carry_s;
}

__global__ __launch_bounds__(kSortThreads) void sort_scatter_kernel(SortPassArgs a) {
  constexpr int W = kSortThreads / 64;
  __shared__ int cnt[W][kSortBuckets];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < W * kSortBuckets; i += kSortThreads) cnt[i / kSortBuckets][i % kSortBuckets] = 0;
  const long long e0 = (long long)blockIdx.x * kSortBlock + (long long)w * 64 * kSortRounds + lane;
  int key[kSortRounds], val[kSortRounds], pos[kSortRounds];
#pragma unroll
  for (int r = 0; r < kSortRounds; ++r) {
    const long long e = e0 + r * 64;
    const bool ok = e < a.n;
    key[r] = ok ? a.keys_in[e] : 0;
    val[r] = ok ? (a.vals_in ? a.vals_in[e] : (int)e) : 0;
  }
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < kSortRounds; ++r) {
    const bool ok = e0 + r * 64 < a.n;
    const int d = sort_digit(key[r], a.shift);
    const unsigned long long peers = sort_peers(d, ok);   // lanes holding the same digit
    const int rank = __builtin_popcountll(peers & lt);
    // the wave's LDS operations complete in issue order: every lane reads the
    // running count before its group's first lane raises it
    const int old = cnt[w][d];
    pos[r] = old + rank;
    if (ok && rank == 0) cnt[w][d] = old + __builtin_popcountll(peers);
  }
  __syncthreads();
  // per digit (one lane each of the first wave): the block's elements of
  // digit d go to block-local positions bstart[d] + (waves before) + rank, and
  // from there to the global start of (d, this block): the totals of the
  // digits below plus this block's offset in row d
  __shared__ int bstart[kSortBuckets], gbase[kSortBuckets];
  if (threadIdx.x < kSortBuckets) {
    const int d = threadIdx.x;
    const int tt = a.tot[d];
    int bt = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) bt += cnt[i][d];
    int x = tt, y = bt;
#pragma unroll
    for (int o = 1; o < kSortBuckets; o <<= 1) {
      const int x2 = __shfl_up(x, o), y2 = __shfl_up(y, o);
      if (d >= o) {
        x += x2;
        y += y2;
      }
    }
    const int bs = y - bt;   // exclusive prefix of the block's digit counts
    bstart[d] = bs;
    gbase[d] = a.hist[(size_t)d * a.B + blockIdx.x] + x - tt;
    int run = bs;
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const int c = cnt[i][d];
      cnt[i][d] = run;
      run += c;
    }
  }
  __syncthreads();
  // stage the block in LDS in its sorted order, then write it out with
  // consecutive lanes on consecutive positions of each digit's run
  __shared__ int ks[kSortBlock], vs[kSortBlock];
#pragma unroll
  for (int r = 0; r < kSortRounds; ++r) {
    if (e0 + r * 64 < a.n) {
      const int p = cnt[w][sort_digit(key[r], a.shift)] + pos[r];
      ks[p] = key[r];
      vs[p] = val[r];
    }
  }
  __syncthreads();
  const long long b0 = (long long)blockIdx.x * kSortBlock;
  const int nvalid = a.n - b0 < kSortBlock ? (int)(a.n - b0) : kSortBlock;
#pragma unroll
  for (int r = 0; r < kSortRounds; ++r) {
    const int i = threadIdx.x + kSortThreads * r;
    if (i < nvalid) {
      const int k = ks[i];
      const int d = sort_digit(k, a.shift);
      const int p = gbase[d] + (i - bstart[d]);
      a.keys_out[p] = k;
      a.vals_out[p] = vs[i];
    }
  }
}

// offsets[e] = first position whose expert is >= e: thread i (0..n) looks at
// the pair (keys[i-1], keys[i]) (keys[-1] = -1, keys[n] = M) and writes every e
// in (keys[i-1], keys[i]]; the ranges are disjoint and cover 0..M.
__global__ __launch_bounds__(256) void sort_offsets_kernel(SortOffsetsArgs a) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i > a.n) return;
  int prev = i > 0 ? a.keys[i - 1] : -1;
  int cur = i < a.n ? a.keys[i] : a.M;
  prev = prev < -1 ? -1 : prev;          // out-of-range experts write nothing outside 0..M
  cur = cur > a.M ? a.M : cur;
  for (int e = prev + 1; e <= cur; ++e) a.offsets[e] = (int)i;
}

hipError_t launch_dispatch_sort(const int* idx, int n, int M, int* sorted_expert, int* sorted_slot,
                                int* offsets, int* hist, int* tmp_keys, int* tmp_vals, hipStream_t stream) {
  const int P = sort_passes(M);
  const int B = (int)(((long long)n + kSortBlock - 1) / kSortBlock);
  const int* kin = idx;
  const int* vin = nullptr;
  for (int p = 0; p < P; ++p) {
    const bool to_out = ((P - 1 - p) & 1) == 0;
    SortPassArgs a;
    a.keys_in = kin;
    a.vals_in = vin;
    a.keys_out = to_out ? sorted_expert : tmp_keys;
    a.vals_out = to_out ? sorted_slot : tmp_vals;
    a.hist = hist;
    a.tot = hist + (size_t)kSortBuckets * B;
    a.n = n;
    a.B = B;
    a.shift = p * kSortDigitBits;
    hipLaunchKernelGGL(sort_hist_kernel, dim3((unsigned)B), dim3(kSortThreads), 0, stream, a);
    hipLaunchKernelGGL(sort_scan_kernel, dim3(kSortBuckets), dim3(kSortScanThreads), 0, stream, hist, hist + (size_t)kSortBuckets * B, B);
    hipLaunchKernelGGL(sort_scatter_kernel, dim3((unsigned)B), dim3(kSortThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    kin = a.keys_out;
    vin = a.vals_out;
  }
  SortOffsetsArgs o;
  o.keys = sorted_expert;
  o.offsets = offsets;
  o.n = n;
  o.M = M;
  hipLaunchKernelGGL(sort_offsets_kernel, dim3((unsigned)(((long long)n + 1 + 255) / 256)), dim3(256), 0, stream, o);
  return hipGetLastError();
}

}  // namespace more
