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
//            a double-buffered group of K-steps in flight (unconditional loads
//            from clamped addresses, so the group really stays in flight), and
//            reads the packed R1 operand (L2-resident).  z stays in registers.
//   split    z -> bf16 hi + bf16 lo (both round to nearest even).  The paper
//            narrows z to bf16 once; keeping the residual makes the logits
//            accurate to ~2^-17 relative, so the selected set is exact except
//            on near-ties far below the logit spread.
//   phase 2  per tile of 32 experts: acc = A_bias x ones (the bias as a bf16
//            hi + lo pair in two K-slots: one extra MFMA per tile instead of
//            64 bytes of bias per lane; -inf on padding rows); acc += R2^T z_hi;
//            acc += R2^T z_lo -> 32 experts x 32 tokens of logits in registers;
//            then the streaming top-k of more_device.h.  The MFMAs of tile t+1
//            are issued before the top-k work on tile t, and the weight
//            operands are fetched two tiles ahead.
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
  const float* biasp;      // fp32 kernels: bias in accumulator layout
  const uint32_t* biasq;   // bf16 kernels: bias as a bf16 hi/lo MFMA operand
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
    // Loads are unconditional (clamped in-bounds addresses) so that the
    // prefetched group stays in flight while the current one is multiplied.
    // Lanes past the last token read a valid row; their results are dropped.
    // In a half-filled last K-step (h % 16 == 8) the upper-half lanes re-read
    // the lower half: the packed R1 rows there are zero.
    constexpr int U = (RB == 1) ? 8 : (RB == 2 ? 4 : 2);  // K-steps per group
    const int KS = (a.h + 15) / 16;
    const long long row = rowok ? n : a.N - 1;
    const uint16_t* xbase = (const uint16_t*)a.X + (size_t)row * a.h;
    const bf16x8* r1p = (const bf16x8*)a.R1p;
    auto xaddr = [&](int s) {
      const int c = (16 * s + 8 * hf < a.h) ? 16 * s + 8 * hf : 16 * s;
      return (const bf16x8*)(xbase + c);
    };
    bf16x8 xa[U], xb[U], ra[U][RB], rb[U][RB];
    auto load = [&](int g, bf16x8 (&xs)[U], bf16x8 (&rs)[U][RB]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = g * U + u;
        xs[u] = __builtin_nontemporal_load(xaddr(s));
#pragma unroll
        for (int b = 0; b < RB; ++b) rs[u][b] = r1p[((size_t)s * RB + b) * kWave + lane];
      }
    };
    auto compute = [&](const bf16x8 (&xs)[U], const bf16x8 (&rs)[U][RB]) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int b = 0; b < RB; ++b) z[b] = mfma_bf16(rs[u][b], xs[u], z[b]);
    };
    const int G = KS / U;                       // full groups
    if (G > 0) {
      // No branch around a load: the group index is clamped instead (a
      // re-load of the last group is harmless), which lets the compiler keep
      // the next group in flight across the loop back-edge.
      load(0, xa, ra);
      int g = 0;
      for (; g + 2 <= G; g += 2) {
        load(g + 1, xb, rb);
        compute(xa, ra);
        load(min(g + 2, G - 1), xa, ra);
        compute(xb, rb);
      }
      if (g < G) compute(xa, ra);
    }
    for (int s = G * U; s < KS; ++s) {          // remainder K-steps
      const bf16x8 xv = __builtin_nontemporal_load(xaddr(s));
#pragma unroll
      for (int b = 0; b < RB; ++b) z[b] = mfma_bf16(r1p[((size_t)s * RB + b) * kWave + lane], xv, z[b]);
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
    // ones in K-slots 0 and 1 of the lower lanes: A_bias x ones puts hi + lo
    // of each expert's bias into every token column.
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (bf16)((!hi && e < 2) ? 1.f : 0.f);
    const bf16x8* r2p = (const bf16x8*)a.R2p;
    const uint32_t* bq = a.biasq;
    struct Ops {
      bf16x8 w[R16];
      uint32_t b;
    };
    auto load_ops = [&](int t, Ops& o) {
      const int tc = t < a.NT ? t : a.NT - 1;   // clamped: always a valid tile
#pragma unroll
      for (int m = 0; m < R16; ++m) o.w[m] = r2p[((size_t)tc * R16 + m) * kWave + lane];
      o.b = bq[(size_t)tc * kWave + lane];
    };
    auto logits = [&](const Ops& o) {
      bf16x8 ab;
#pragma unroll
      for (int e = 0; e < 8; ++e) ab[e] = (bf16)0.f;
      const uint32_t bw = o.b;
      ab[0] = __builtin_bit_cast(bf16, (uint16_t)(bw & 0xffffu));
      ab[1] = __builtin_bit_cast(bf16, (uint16_t)(bw >> 16));
      floatx16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
      acc = mfma_bf16(ab, ones, acc);
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(o.w[m], zh[m], acc);
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(o.w[m], zl[m], acc);
      return acc;
    };
    // Two tiles in flight: the MFMAs of tile t+1 are issued before the top-k
    // work on tile t, and operands are fetched two tiles ahead.
    Ops o0, o1;
    load_ops(0, o0);
    load_ops(1, o1);
    floatx16 accA = logits(o0);
    load_ops(2, o0);
    for (int t = 0; t < a.NT; t += 2) {
      floatx16 accB = logits(o1);
      load_ops(t + 3, o1);
      st.template tile<FULL>(accA, kTile * t + 4 * hf, lg, lane, hi, a.perm, a.k);
      accA = logits(o0);                        // beyond the last tile: unused
      load_ops(t + 4, o0);
      if (t + 1 < a.NT) st.template tile<FULL>(accB, kTile * (t + 1) + 4 * hf, lg, lane, hi, a.perm, a.k);
    }
  } else {
    constexpr int KS2 = 8 * R16;
    const floatx16* biasp = (const floatx16*)a.biasp;      // [NT][2] x 16 floats
    const float* r2p = (const float*)a.R2p;
    for (int t = 0; t < a.NT; ++t) {
      floatx16 acc = biasp[2 * t + hf];
#pragma unroll
      for (int m = 0; m < KS2; ++m)
        acc = mfma_f32(r2p[((size_t)t * KS2 + m) * kWave + lane], z[m >> 4][m & 15], acc);
      st.template tile<FULL>(acc, kTile * t + 4 * hf, lg, lane, hi, a.perm, a.k);
    }
  }

  finish_tokens<KMAX, CAP, FULL>(st, lg, lane, hi, rowok, n, a.perm, a.k, a.out_idx, a.out_gate,
                                 a.out_logit, a.out_lse);
}

}  // namespace more
