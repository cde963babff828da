// more_lowrank.h -- fused low-rank router + top-k + gates for gfx950.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.1 Algorithm 1 (phase 1: z = X-block times the
// down-projection accumulated on chip; phase 2: one sweep over the experts
// with a running top-k; only the N x k results are written), Fig. 12 (gates
// are a softmax over the k selected logits) and App. F.2.1 eq. (6)/(8) (full
// softmax via a running maximum and normaliser).
//
// One wave owns 32 tokens; there is no cross-wave communication and no
// barrier.  Per wave:
//   phase 1  z^T (r x 32) = R1^T X^T with v_mfma_f32_32x32x16_bf16: each lane
//            streams 16 bytes of one X row per K-step (16 hidden units), with
//            a double-buffered group of K-steps in flight, and reads the
//            packed R1 operand (L2-resident).  z stays in the accumulators.
//   split    z -> bf16 hi + bf16 lo (both round to nearest even).  The paper
//            narrows z to bf16 once; keeping the residual makes the logits
//            accurate to ~2^-17 relative, so the selected set is exact except
//            on near-ties far below the logit spread.
//   phase 2  per tile of 32 experts: acc = bias (C operand, -inf on padding);
//            acc += R2^T z_hi; acc += R2^T z_lo  -> 32 experts x 32 tokens of
//            logits in registers; then the streaming top-k of more_device.h.
//   end      merge the two half-token logs, order by (logit desc, expert
//            index asc), form the gates, store.
#pragma once
#include "more_device.h"
#include "more_pack.h"

namespace more {

struct LowRankArgs {
  const void* X;
  long long N;
  int h;
  int NT;          // expert tiles of 32
  int k;
  const void* R1p;
  const void* R2p;
  const float* biasp;
  const int* perm;
  int* out_idx;
  float* out_gate;
  float* out_logit;   // may be null
  float* out_lse;     // may be null
};

template <int KMAX> struct Cap { static constexpr int value = 2 * KMAX + 8; };

template <int DT, int KMAX, bool FULL, int R16, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void lowrank_kernel(LowRankArgs a) {
  constexpr int CAP = Cap<KMAX>::value;
  constexpr int RB = (R16 + 1) / 2;                        // 32-row blocks of z
  extern __shared__ float2 smem_log[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool hi = lane >= 32;
  const int hf = hi ? 1 : 0, col = lane & 31;
  const long long tok0 = ((long long)blockIdx.x * WAVES + wave) * kTile;
  if (tok0 >= a.N) return;                                  // wave-uniform
  const long long n = tok0 + col;
  const bool rowok = n < a.N;
  LogRef lg{smem_log + (size_t)wave * CAP * kWave};

  // ------------------------------------------------------------------ phase 1
  floatx16 z[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) z[b][v] = 0.f;

  if constexpr (DT == 0) {
    constexpr int U = (RB == 1) ? 8 : (RB == 2 ? 4 : 2);  // K-steps per group
    const int KS = (a.h + 15) / 16;
    const bf16x8* xrow = (const bf16x8*)((const uint16_t*)a.X + (size_t)(rowok ? n : tok0) * a.h + 8 * hf);
    const bf16x8* r1p = (const bf16x8*)a.R1p;
    bf16x8 xa[U], xb[U], ra[U][RB], rb[U][RB];
    auto load = [&](int g, bf16x8 (&xs)[U], bf16x8 (&rs)[U][RB]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = g * U + u;
        bf16x8 xv;
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = (bf16)0.f;
        if (rowok && s < KS && 16 * s + 8 * hf < a.h) xv = __builtin_nontemporal_load(xrow + 2 * s);
        xs[u] = xv;
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          bf16x8 rv;
#pragma unroll
          for (int e = 0; e < 8; ++e) rv[e] = (bf16)0.f;
          if (s < KS) rv = r1p[((size_t)s * RB + b) * kWave + lane];
          rs[u][b] = rv;
        }
      }
    };
    auto compute = [&](const bf16x8 (&xs)[U], const bf16x8 (&rs)[U][RB]) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int b = 0; b < RB; ++b) z[b] = mfma_bf16(rs[u][b], xs[u], z[b]);
    };
    const int G = (KS + U - 1) / U;
    load(0, xa, ra);
    for (int g = 0; g < G; g += 2) {
      if (g + 1 < G) load(g + 1, xb, rb);
      compute(xa, ra);
      if (g + 1 < G) {
        if (g + 2 < G) load(g + 2, xa, ra);
        compute(xb, rb);
      }
    }
  } else {
    const int KS = (a.h + 1) / 2;
    const float* xrow = (const float*)a.X + (size_t)(rowok ? n : tok0) * a.h + hf;
    const float* r1p = (const float*)a.R1p;
    for (int s = 0; s < KS; ++s) {
      const float xv = (rowok && 2 * s + hf < a.h) ? xrow[2 * s] : 0.f;
#pragma unroll
      for (int b = 0; b < RB; ++b) z[b] = mfma_f32(r1p[((size_t)s * RB + b) * kWave + lane], xv, z[b]);
    }
  }

  // ------------------------------------------------------------------ phase 2
  SweepState<KMAX, CAP> st;
  st.init(a.k);
  const floatx16* biasp = (const floatx16*)a.biasp;        // [NT][2] x 16 floats
  if constexpr (DT == 0) {
    bf16x8 zh[R16], zl[R16];
#pragma unroll
    for (int m = 0; m < R16; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = z[m >> 1][8 * (m & 1) + e];
        const bf16 hv = (bf16)f;
        zh[m][e] = hv;
        zl[m][e] = (bf16)(f - (float)hv);
      }
    const bf16x8* r2p = (const bf16x8*)a.R2p;
    floatx16 bc = biasp[hf];
    bf16x8 a2[R16];
#pragma unroll
    for (int m = 0; m < R16; ++m) a2[m] = r2p[(size_t)m * kWave + lane];
    for (int t = 0; t < a.NT; ++t) {
      floatx16 acc = bc;
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(a2[m], zh[m], acc);
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(a2[m], zl[m], acc);
      if (t + 1 < a.NT) {
        bc = biasp[2 * (t + 1) + hf];
#pragma unroll
        for (int m = 0; m < R16; ++m) a2[m] = r2p[((size_t)(t + 1) * R16 + m) * kWave + lane];
      }
      st.template tile<FULL>(acc, kTile * t + 4 * hf, lg, lane, hi, a.perm, a.k);
    }
  } else {
    constexpr int KS2 = 8 * R16;
    const float* r2p = (const float*)a.R2p;
    for (int t = 0; t < a.NT; ++t) {
      floatx16 acc = biasp[2 * t + hf];
#pragma unroll
      for (int m = 0; m < KS2; ++m)
        acc = mfma_f32(r2p[((size_t)t * KS2 + m) * kWave + lane], z[m >> 4][m & 15], acc);
      st.template tile<FULL>(acc, kTile * t + 4 * hf, lg, lane, hi, a.perm, a.k);
    }
  }

  // ------------------------------------------------------------------ merge
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
