// Merge of per-shard top-k candidate lists: kernel and launch.
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. E.3, Fig. 12, eq. (6) / (8).
#include "more_device.h"
#include "more_merge.h"

namespace more {

// One lane per token.  The list keeps KMAX slots, the first KMAX - k of them
// +inf fillers, so its k-th best is always slot KMAX - 1.  Each shard list is
// ordered by logit descending, so a shard is left at its first entry below
// the current k-th (a tie may still win on the expert index and is offered
// to the ordered insert, which keeps (logit desc, global index asc)).
template <int KMAX, bool FULL>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const long long n = (long long)blockIdx.x * 256 + threadIdx.x;
  if (n >= a.N) return;
  float V[KMAX];
  int IX[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    V[j] = (j < KMAX - a.k) ? __builtin_inff() : -__builtin_inff();
    IX[j] = (j < KMAX - a.k) ? -1 : 0x7fffffff;
  }
  for (int g = 0; g < a.G; ++g) {
    const size_t base = ((size_t)g * a.N + n) * a.k;
    const long long off = (long long)g * a.W;
    for (int j = 0; j < a.k; ++j) {
      const float x = a.cand_logit[base + j];
      if (x < V[KMAX - 1]) break;
      ordered_insert<KMAX>(V, IX, x, (int)(off + a.cand_idx[base + j]));
    }
  }
  float lse = 0.f;
  if (FULL) {
    // eq. (8) across the shards: log of the sum of the shard normalisers
    float mm = -__builtin_inff();
    for (int g = 0; g < a.G; ++g) mm = fmaxf(mm, a.shard_lse[(size_t)g * a.N + n]);
    float z = 0.f;
    for (int g = 0; g < a.G; ++g) z += __builtin_amdgcn_exp2f((a.shard_lse[(size_t)g * a.N + n] - mm) * kLog2e);
    lse = mm + __builtin_amdgcn_logf(z) * kLn2;
  }
  // the best selected logit: slot KMAX - k (read without a dynamic index)
  float vmax = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j == KMAX - a.k) vmax = V[j];
  float w[KMAX];
  float denom = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool real = j >= KMAX - a.k;
    w[j] = real ? __builtin_amdgcn_exp2f((V[j] - (FULL ? lse : vmax)) * kLog2e) : 0.f;
    denom += w[j];
  }
  const float inv = FULL ? 1.f : 1.f / denom;
  const size_t o = (size_t)n * a.k;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j >= KMAX - a.k) {
      const int t = j - (KMAX - a.k);
      a.out_idx[o + t] = IX[j];
      a.out_gate[o + t] = w[j] * inv;
      if (a.out_logit) a.out_logit[o + t] = V[j];
    }
  }
  if (FULL && a.out_lse) a.out_lse[n] = lse;
}

template <int KMAX>
static hipError_t launch_k(const MergeArgs& a, bool full, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + 255) / 256));
  if (full)
    hipLaunchKernelGGL((merge_kernel<KMAX, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((merge_kernel<KMAX, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk_merge(const MergeArgs& a, bool full, hipStream_t stream) {
  if (a.k <= 4) return launch_k<4>(a, full, stream);
  if (a.k <= 8) return launch_k<8>(a, full, stream);
  if (a.k <= 16) return launch_k<16>(a, full, stream);
  return launch_k<32>(a, full, stream);
}

}  // namespace more
