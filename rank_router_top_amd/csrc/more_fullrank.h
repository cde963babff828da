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

  finish_tokens<KMAX, CAP, FULL>(st, lg, lane, hi, rowok, n, a.perm, a.k, a.out_idx, a.out_gate,
                                 a.out_logit, a.out_lse);
}

}  // namespace more
