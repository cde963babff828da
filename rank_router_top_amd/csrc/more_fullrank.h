// more_fullrank.h -- fused standard (full-rank) router + top-k + gates for gfx950.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", §2 (standard router softmax(TopK(R x))) fused the same way as the
// low-rank kernel (App. H.3, Fig. 20: no N x M logits in memory, but each
// expert tile needs the full h-long weight columns instead of a rank-r
// intermediate).
//
// One wave owns 32 tokens and sweeps all expert tiles; each 32x32 logit tile
// is a K = h reduction of v_mfma_f32_32x32x16_bf16 (A = packed W^T tile, B =
// the wave's X rows), then the same streaming top-k as the low-rank kernel.
#pragma once
#include "more_device.h"
#include "more_pack.h"

namespace more {

struct FullRankArgs {
  const void* X;
  long long N;
  int h;
  int NT;
  int k;
  int KSW;            // K-steps over h
  const void* Wp;     // [NT][KSW][64][EPL]
  const float* biasp;
  const int* perm;
  int* out_idx;
  float* out_gate;
  float* out_logit;
  float* out_lse;
};

template <int DT, int KMAX, bool FULL, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void fullrank_kernel(FullRankArgs a) {
  constexpr int CAP = 2 * KMAX + 8;
  extern __shared__ float2 smem_log[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool hi = lane >= 32;
  const int hf = hi ? 1 : 0, col = lane & 31;
  const long long tok0 = ((long long)blockIdx.x * WAVES + wave) * kTile;
  if (tok0 >= a.N) return;
  const long long n = tok0 + col;
  const bool rowok = n < a.N;
  LogRef lg{smem_log + (size_t)wave * CAP * kWave};
  const floatx16* biasp = (const floatx16*)a.biasp;

  SweepState<KMAX, CAP> st;
  st.init(a.k);
  if constexpr (DT == 0) {
    const bf16x8* xrow = (const bf16x8*)((const uint16_t*)a.X + (size_t)(rowok ? n : tok0) * a.h + 8 * hf);
    const bf16x8* wp = (const bf16x8*)a.Wp;
    for (int t = 0; t < a.NT; ++t) {
      floatx16 acc = biasp[2 * t + hf];
      for (int s = 0; s < a.KSW; ++s) {
        bf16x8 xv;
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = (bf16)0.f;
        if (rowok && 16 * s + 8 * hf < a.h) xv = xrow[2 * s];
        acc = mfma_bf16(wp[((size_t)t * a.KSW + s) * kWave + lane], xv, acc);
      }
      st.template tile<FULL>(acc, kTile * t + 4 * hf, lg, lane, hi, a.perm, a.k);
    }
  } else {
    const float* xrow = (const float*)a.X + (size_t)(rowok ? n : tok0) * a.h + hf;
    const float* wp = (const float*)a.Wp;
    for (int t = 0; t < a.NT; ++t) {
      floatx16 acc = biasp[2 * t + hf];
      for (int s = 0; s < a.KSW; ++s) {
        const float xv = (rowok && 2 * s + hf < a.h) ? xrow[2 * s] : 0.f;
        acc = mfma_f32(wp[((size_t)t * a.KSW + s) * kWave + lane], xv, acc);
      }
      st.template tile<FULL>(acc, kTile * t + 4 * hf, lg, lane, hi, a.perm, a.k);
    }
  }

  st.thr_p = partner_f32(st.L[KMAX - 1], hi);
  st.thr = fmaxf(st.L[KMAX - 1], st.thr_p);
  st.compact(lg, lane, a.perm, a.k);
  const int cnt_p = (int)partner_u32((uint32_t)st.cnt, hi);
  float lse = 0.f;
  if (FULL) {
    const float mp = partner_f32(st.m, hi), Zp = partner_f32(st.Z, hi);
    const float mm = fmaxf(st.m, mp);
    const float Zt = st.Z * __builtin_amdgcn_exp2f((st.m - mm) * kLog2e) +
                     Zp * __builtin_amdgcn_exp2f((mp - mm) * kLog2e);
    lse = mm + __builtin_amdgcn_logf(Zt) * kLn2;
  }
  if (hi || !rowok) return;
  float V[KMAX];
  int IX[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    V[j] = -__builtin_inff();
    IX[j] = 0x7fffffff;
  }
  for (int c = 0; c < st.cnt; ++c) {
    const float2 e = lg.base[c * kWave + lane];
    ordered_insert<KMAX>(V, IX, e.x, a.perm[__float_as_int(e.y)]);
  }
  for (int c = 0; c < cnt_p; ++c) {
    const float2 e = lg.base[c * kWave + lane + 32];
    ordered_insert<KMAX>(V, IX, e.x, a.perm[__float_as_int(e.y)]);
  }
  float w[KMAX];
  if (FULL) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) w[j] = __builtin_amdgcn_exp2f((V[j] - lse) * kLog2e);
  } else {
    float denom = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      w[j] = (j < a.k) ? __builtin_amdgcn_exp2f((V[j] - V[0]) * kLog2e) : 0.f;
      denom += w[j];
    }
    const float inv = 1.f / denom;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) w[j] *= inv;
  }
  const size_t o = (size_t)n * a.k;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < a.k) {
      a.out_idx[o + j] = IX[j];
      a.out_gate[o + j] = w[j];
      if (a.out_logit) a.out_logit[o + j] = V[j];
    }
  }
  if (FULL && a.out_lse) a.out_lse[n] = lse;
}

}  // namespace more
