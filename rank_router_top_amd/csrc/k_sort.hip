// Expert dispatch sort + count: kernels and launch.
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. E, Fig. 9 (sort + count after the router).
#include "more_sort.h"

namespace more {

__device__ __forceinline__ int sort_digit(int key, int shift) { return (int)(((unsigned)key >> shift) & (kSortBuckets - 1)); }

__global__ __launch_bounds__(kSortThreads) void sort_hist_kernel(SortPassArgs a) {
  __shared__ int h[kSortBuckets];
  if (threadIdx.x < kSortBuckets) h[threadIdx.x] = 0;
  __syncthreads();
  const long long e0 = (long long)blockIdx.x * kSortBlock;
  for (int i = threadIdx.x; i < kSortBlock; i += kSortThreads) {
    const long long e = e0 + i;
    if (e < a.n) atomicAdd(&h[sort_digit(a.keys_in[e], a.shift)], 1);
  }
  __syncthreads();
  if (threadIdx.x < kSortBuckets) a.hist[(size_t)threadIdx.x * a.B + blockIdx.x] = h[threadIdx.x];
}

// One workgroup: in-place exclusive scan of the 64 * B counts.
__global__ __launch_bounds__(kSortScanThreads) void sort_scan_kernel(int* hist, int total) {
  __shared__ int part[kSortScanThreads];
  const int per = (total + kSortScanThreads - 1) / kSortScanThreads;
  const int lo = threadIdx.x * per;
  const int hi = lo + per < total ? lo + per : total;
  int s = 0;
  for (int i = lo; i < hi; ++i) s += hist[i];
  part[threadIdx.x] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the per-thread sums
  for (int o = 1; o < kSortScanThreads; o <<= 1) {
    const int v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = part[threadIdx.x] - s;   // exclusive prefix of this thread's range
  for (int i = lo; i < hi; ++i) {
    const int c = hist[i];
    hist[i] = run;
    run += c;
  }
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
    // lanes holding the same digit: intersect the six bit ballots
    unsigned long long peers = __builtin_amdgcn_ballot_w64(ok);
#pragma unroll
    for (int bit = 0; bit < kSortDigitBits; ++bit) {
      const unsigned long long b = __builtin_amdgcn_ballot_w64(((d >> bit) & 1) != 0);
      peers &= ((d >> bit) & 1) ? b : ~b;
    }
    const int rank = __builtin_popcountll(peers & lt);
    // the wave's LDS operations complete in issue order: every lane reads the
    // running count before its group's first lane raises it
    const int old = cnt[w][d];
    pos[r] = old + rank;
    if (ok && rank == 0) cnt[w][d] = old + __builtin_popcountll(peers);
  }
  __syncthreads();
  // per digit: this block's base, then each wave's start after the waves before it
  if (threadIdx.x < kSortBuckets) {
    int run = a.hist[(size_t)threadIdx.x * a.B + blockIdx.x];
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const int c = cnt[i][threadIdx.x];
      cnt[i][threadIdx.x] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSortRounds; ++r) {
    if (e0 + r * 64 < a.n) {
      const int p = cnt[w][sort_digit(key[r], a.shift)] + pos[r];
      a.keys_out[p] = key[r];
      a.vals_out[p] = val[r];
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
    a.n = n;
    a.B = B;
    a.shift = p * kSortDigitBits;
    hipLaunchKernelGGL(sort_hist_kernel, dim3((unsigned)B), dim3(kSortThreads), 0, stream, a);
    hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(kSortScanThreads), 0, stream, hist, kSortBuckets * B);
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
