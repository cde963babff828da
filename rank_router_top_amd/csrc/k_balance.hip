// Balancing statistics of the training forward: kernel instances and launch.
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.2.1 (eq. 6, 7, 9; Algorithm 2, second sweep) and App. G.1.
#include "more_balance.h"

namespace more {

// Grid: slots * ceil(M / kCountBins) workgroups of kCountThreads threads;
// workgroup (s, e) counts the entries of blocks s, s + slots, ... that fall
// in experts e * kCountBins .. + kCountBins - 1.
__global__ __launch_bounds__(kCountThreads) void count_kernel(CountArgs a) {
  __shared__ int hist[kCountBins];
  const int E = (a.M + kCountBins - 1) / kCountBins;
  const int s = blockIdx.x / E, e = blockIdx.x % E;
  const int lo = e * kCountBins;
  const int nb = a.M - lo < kCountBins ? a.M - lo : kCountBins;
  for (int i = threadIdx.x; i < nb; i += kCountThreads) hist[i] = 0;
  __syncthreads();
  const long long total = a.N * a.k;
  const int per = kTile * a.k;   // entries of one 32-token block
  for (long long j = s; j < a.NB; j += a.slots) {
    const long long b0 = j * per;
    for (int i = threadIdx.x; i < per; i += kCountThreads) {
      if (b0 + i < total) {
        const int x = a.idx[b0 + i] - lo;
        if (x >= 0 && x < nb) atomicAdd(&hist[x], 1);
      }
    }
  }
  __syncthreads();
  int* row = a.cpart + (size_t)s * a.M + lo;
  for (int i = threadIdx.x; i < nb; i += kCountThreads) row[i] = hist[i];
}


// Grid: ceil(Mpad / 32) workgroups of 256 threads.  Workgroup b owns columns
// 32b .. 32b + 31; thread (c, q) = (tid % 32, tid / 32) sums slots q, q + 8, ...
// of column 32b + c, and the eight partial sums are added in order q = 0..7,
// so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void colsum_kernel(ColsumArgs a) {
  __shared__ float fp[8][32];
  __shared__ int cp[8][32];
  const int c = threadIdx.x & 31, q = threadIdx.x >> 5;
  const int p = blockIdx.x * 32 + c;
  float sp = 0.f;
  int sc = 0;
  if (p < a.Mpad) {
#pragma unroll 8
    for (int s = q; s < a.slots; s += 8) sp += a.part[(size_t)s * a.Mpad + p];
  }
  if (p < a.M) {
#pragma unroll 8
    for (int s = q; s < a.slots; s += 8) sc += a.cpart[(size_t)s * a.M + p];
  }
  fp[q][c] = sp;
  cp[q][c] = sc;
  __syncthreads();
  if (q != 0 || p >= a.Mpad) return;
  float tp = 0.f;
  int tc = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    tp += fp[i][c];
    tc += cp[i][c];
  }
  const int ex = a.perm[p];
  if (ex >= 0 && ex < a.M) a.psum[ex] = tp;
  if (p < a.M) a.counts[p] = tc;
}

// One workgroup of 1024 threads.  With c_i the counts and C = N k:
//   L_bal = M sum_i (c_i / C) (psum_i / N)
//   H_norm = (log C - (1/C) sum_{c_i > 0} c_i log c_i) / log M   (1 for M = 1)
__global__ __launch_bounds__(1024) void stats_kernel(StatsArgs a) {
  __shared__ double red[2][1024 / kWave];
  double sl = 0.0, sh = 0.0;
  for (int i = threadIdx.x; i < a.M; i += 1024) {
    const double c = (double)a.counts[i];
    sl += c * (double)a.psum[i];
    if (c > 0.0) sh += c * log(c);
  }
  for (int o = 32; o >= 1; o >>= 1) {
    sl += __shfl_xor(sl, o);
    sh += __shfl_xor(sh, o);
  }
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wv] = sl;
    red[1][wv] = sh;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double tl = 0.0, th = 0.0;
    for (int i = 0; i < 1024 / kWave; ++i) {
      tl += red[0][i];
      th += red[1][i];
    }
    const double C = (double)a.N * (double)a.k;
    const double lbal = (double)a.M * tl / (C * (double)a.N);
    const double hn = a.M > 1 ? (log(C) - th / C) / log((double)a.M) : 1.0;
    a.stats[0] = (float)lbal;
    a.stats[1] = (float)hn;
  }
}

hipError_t launch_balance(int r16, const PsumArgs& pa, const CountArgs& ca, const ColsumArgs& sa,
                          const StatsArgs& ta, hipStream_t stream) {
  const dim3 pg((unsigned)(pa.slots * pa.G)), pb(64 * kBalWaves);
  switch (r16) {
    case 1: hipLaunchKernelGGL((psum_kernel<1, bal_tiles(1), kBalWaves>), pg, pb, 0, stream, pa); break;
    case 2: hipLaunchKernelGGL((psum_kernel<2, bal_tiles(2), kBalWaves>), pg, pb, 0, stream, pa); break;
    default: hipLaunchKernelGGL((psum_kernel<4, bal_tiles(4), kBalWaves>), pg, pb, 0, stream, pa); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int E = (ca.M + kCountBins - 1) / kCountBins;
  hipLaunchKernelGGL(count_kernel, dim3((unsigned)(ca.slots * E)), dim3(kCountThreads), 0, stream, ca);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)((sa.Mpad + 31) / 32)), dim3(256), 0, stream, sa);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(1024), 0, stream, ta);
  return hipGetLastError();
}

}  // namespace more
