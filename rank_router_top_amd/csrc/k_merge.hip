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

// k == KMAX (4, 8 or 16) with 16-byte aligned candidate arrays: a lane
// reads its token's lists with 16-byte loads, the next shard's while it
// merges the current one.
template <int KMAX, bool FULL>
__global__ __launch_bounds__(256) void merge_vec_kernel(MergeArgs a) {
  constexpr int C = KMAX / 4;
  const long long n = (long long)blockIdx.x * 256 + threadIdx.x;
  if (n >= a.N) return;
  float V[KMAX];
  int IX[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    V[j] = -__builtin_inff();
    IX[j] = 0x7fffffff;
  }
  float4 lc[C], ln[C];
  int4 ic[C], in_[C];
  auto load = [&](int g, float4 (&l)[C], int4 (&ix)[C]) {
    const size_t base = ((size_t)g * a.N + n) * KMAX;
    const float4* lp = (const float4*)(a.cand_logit + base);
    const int4* ip = (const int4*)(a.cand_idx + base);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      l[c] = lp[c];
      ix[c] = ip[c];
    }
  };
  load(0, lc, ic);
  for (int g = 0; g < a.G; ++g) {
    if (g + 1 < a.G) load(g + 1, ln, in_);
    const int off = (int)((long long)g * a.W);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float x[4] = {lc[c].x, lc[c].y, lc[c].z, lc[c].w};
      const int ix[4] = {ic[c].x, ic[c].y, ic[c].z, ic[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (x[e] >= V[KMAX - 1]) ordered_insert<KMAX>(V, IX, x[e], off + ix[e]);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      lc[c] = ln[c];
      ic[c] = in_[c];
    }
  }
  float lse = 0.f;
  if (FULL) {
    float mm = -__builtin_inff();
    for (int g = 0; g < a.G; ++g) mm = fmaxf(mm, a.shard_lse[(size_t)g * a.N + n]);
    float z = 0.f;
    for (int g = 0; g < a.G; ++g) z += __builtin_amdgcn_exp2f((a.shard_lse[(size_t)g * a.N + n] - mm) * kLog2e);
    lse = mm + __builtin_amdgcn_logf(z) * kLn2;
  }
  float w[KMAX];
  float denom = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    w[j] = __builtin_amdgcn_exp2f((V[j] - (FULL ? lse : V[0])) * kLog2e);
    denom += w[j];
  }
  const float inv = FULL ? 1.f : 1.f / denom;
  float4* og = (float4*)(a.out_gate + (size_t)n * KMAX);
  int4* oi = (int4*)(a.out_idx + (size_t)n * KMAX);
  float4* ol = a.out_logit ? (float4*)(a.out_logit + (size_t)n * KMAX) : nullptr;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    oi[c] = make_int4(IX[4 * c], IX[4 * c + 1], IX[4 * c + 2], IX[4 * c + 3]);
    og[c] = make_float4(w[4 * c] * inv, w[4 * c + 1] * inv, w[4 * c + 2] * inv, w[4 * c + 3] * inv);
    if (ol) ol[c] = make_float4(V[4 * c], V[4 * c + 1], V[4 * c + 2], V[4 * c + 3]);
  }
  if (FULL && a.out_lse) a.out_lse[n] = lse;
}

// Many shards (G >= 32): one wave per token.  Lane l merges shards l, l + 64,
// ... into its own ordered list; then k rounds each take the best head over
// the wave (logit desc, index asc) and pop it from its lane.  The
// full-softmax normaliser combines the lanes' shard values with a butterfly
// (eq. (8)); the order of every sum is fixed.
template <int KMAX, bool FULL>
__global__ __launch_bounds__(256) void merge_wave_kernel(MergeArgs a) {
  __shared__ float mw_lv[4][KMAX * kWave];   // per wave: the lanes' merged lists, [entry][lane]
  __shared__ int mw_li[4][KMAX * kWave];
  const int lane = threadIdx.x & 63;
  const long long n = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= a.N) return;   // wave-uniform
  float V[KMAX];
  int IX[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    V[j] = -__builtin_inff();
    IX[j] = 0x7fffffff;
  }
  float m = -__builtin_inff(), Z = 0.f;
  // whole lists as 16-byte loads when every list is KMAX entries on a 16-byte boundary
  const bool vec = a.k == KMAX && (KMAX % 4) == 0 && (((uintptr_t)a.cand_logit | (uintptr_t)a.cand_idx) & 15) == 0;
  // lane l takes shards l, l + 64, ...: the first list as it is (each shard's
  // list is ordered by (logit desc, index asc)), every further one by a
  // bitonic top-KMAX merge
  for (int it = 0; it * kWave < a.G; ++it) {
    const int g = lane + it * kWave;
    const bool gok = g < a.G;
    const size_t base = ((size_t)(gok ? g : 0) * a.N + n) * a.k;
    const long long off = (long long)g * a.W;
    float cl[KMAX];
    int ci[KMAX];
    if (vec) {
#pragma unroll
      for (int q = 0; q < KMAX / 4; ++q) {
        const float4 x = ((const float4*)(a.cand_logit + base))[q];
        const int4 y = ((const int4*)(a.cand_idx + base))[q];
        cl[4 * q] = x.x, cl[4 * q + 1] = x.y, cl[4 * q + 2] = x.z, cl[4 * q + 3] = x.w;
        ci[4 * q] = y.x, ci[4 * q + 1] = y.y, ci[4 * q + 2] = y.z, ci[4 * q + 3] = y.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        cl[j] = j < a.k ? a.cand_logit[base + j] : -__builtin_inff();
        ci[j] = j < a.k ? a.cand_idx[base + j] : 0;
      }
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool real = gok && j < a.k;
      cl[j] = real ? cl[j] : -__builtin_inff();
      ci[j] = real ? (int)(off + ci[j]) : 0x7fffffff;
    }
    if (it == 0) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        V[j] = cl[j];
        IX[j] = ci[j];
      }
    } else {
      bitonic_top<KMAX>(V, IX, cl, ci);
    }
    if (FULL && gok) {
      const float l = a.shard_lse[(size_t)g * a.N + n];
      const float mn = fmaxf(m, l);
      Z = Z * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + __builtin_amdgcn_exp2f((l - mn) * kLog2e);
      m = mn;
    }
  }
  float lse = 0.f;
  if (FULL) {
    float mm = m;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o));
    float z = m > -__builtin_inff() ? Z * __builtin_amdgcn_exp2f((m - mm) * kLog2e) : 0.f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o);
    lse = mm + __builtin_amdgcn_logf(z) * kLn2;
  }
  // k rounds: the wave's best head, popped from the lane that holds it.  The
  // best of each 16-lane row by DPP (quad swaps, then rotations by 4 and 8
  // within the row), then of the four rows' results read into scalars.  The
  // lane's list waits in LDS; only the lane that gave up its head reads the
  // next entry.
  float* lv = mw_lv[threadIdx.x >> 6];
  int* li = mw_li[threadIdx.x >> 6];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    lv[j * kWave + lane] = V[j];
    li[j * kWave + lane] = IX[j];
  }
  float hv = V[0];
  int hx = IX[0], h = 0;
  float rv = -__builtin_inff();   // lane j keeps round j's logit and index
  int ri = 0x7fffffff;
  auto take = [](float& v, int& i, float v2, int i2) {
    const bool better = ahead(v2, i2, v, i);
    v = better ? v2 : v;
    i = better ? i2 : i;
  };
  for (int r = 0; r < a.k; ++r) {
    float v = hv;
    int i = hx;
#define MORE_DPP_STEP(ctrl)                                                                                   \
  take(v, i, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), ctrl, 0xf, 0xf, false)), \
       __builtin_amdgcn_update_dpp(i, i, ctrl, 0xf, 0xf, false))
    MORE_DPP_STEP(0xB1);    // quad_perm [1,0,3,2]
    MORE_DPP_STEP(0x4E);    // quad_perm [2,3,0,1]
    MORE_DPP_STEP(0x124);   // row_ror:4
    MORE_DPP_STEP(0x128);   // row_ror:8
#undef MORE_DPP_STEP
    float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int row = 1; row < 4; ++row)
      take(bv, bi, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * row)),
           __builtin_amdgcn_readlane(i, 16 * row));
    if (lane == r) {
      rv = bv;
      ri = bi;
    }
    if (hv == bv && hx == bi) {   // the lane that held it (several only for exhausted lists)
      ++h;
      hv = h < KMAX ? lv[h * kWave + lane] : -__builtin_inff();
      hx = h < KMAX ? li[h * kWave + lane] : 0x7fffffff;
    }
  }
  // gates: round 0 holds the best logit
  const float v0 = __shfl(rv, 0);
  const float w = lane < a.k ? __builtin_amdgcn_exp2f((rv - (FULL ? lse : v0)) * kLog2e) : 0.f;
  float denom = w;
  if (!FULL) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) denom += __shfl_xor(denom, o);
  }
  if (lane < a.k) {
    const size_t o = (size_t)n * a.k + lane;
    a.out_idx[o] = ri;
    a.out_gate[o] = FULL ? w : w / denom;
    if (a.out_logit) a.out_logit[o] = rv;
  }
  if (FULL && a.out_lse && lane == 0) a.out_lse[n] = lse;
}

static bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15) == 0; }

template <int KMAX>
static hipError_t launch_k(const MergeArgs& a, bool full, hipStream_t s) {
  if (a.G >= 32 && a.N <= (1LL << 30)) {
    const dim3 wgrid((unsigned)((a.N + 3) / 4));
    if (full)
      hipLaunchKernelGGL((merge_wave_kernel<KMAX, true>), wgrid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((merge_wave_kernel<KMAX, false>), wgrid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((a.N + 255) / 256));
  if constexpr (KMAX <= 16) {   // larger lists spill in the 16-byte form
    const bool vec = a.k == KMAX && aligned16(a.cand_logit) && aligned16(a.cand_idx) && aligned16(a.out_idx) &&
                     aligned16(a.out_gate) && aligned16(a.out_logit);
    if (vec) {
      if (full)
        hipLaunchKernelGGL((merge_vec_kernel<KMAX, true>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((merge_vec_kernel<KMAX, false>), grid, dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
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
