// more_stream.h -- persistent, streaming form of the fused low-rank router
// (bf16 storage, r <= 64) for gfx950.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.1 Algorithm 1: per token block, phase 1 (z = X-block times
// the down-projection, on chip) then phase 2 (one sweep over the experts with
// a running top-k).  The paper runs the two phases back to back inside one
// program per block.  On MI355X that leaves HBM idle while a block sweeps
// and the vector units idle while it streams X, so here every wave is
// persistent, owns several 32-token blocks, and overlaps the two phases of
// consecutive blocks:
//
//     sweep block i (VALU + MFMA)   ||   stream X of block i+1 into z (HBM + MFMA)
//
// The X stream runs through a ring of D register slots (one 16-byte load per
// lane per K-step, issued D K-steps ahead).  The K-steps of block i+1 are done
// in batches of D, each batch followed by its share of block i's expert
// tiles, so X keeps flowing while the tiles are processed.  The sweep itself
// is two tiles deep: the MFMAs of tile t+1 are issued before the top-k work
// on tile t, and weight operands arrive two tiles ahead; the operand
// pipeline wraps from the last tile of a block to the first tile of the next.
//
// No load sits under a branch: loads that have no work (past the last block,
// padded K-steps) read a fixed cache-resident address instead, which keeps
// the compiler's wait counts exact and costs no HBM traffic.
#pragma once
#include "more_device.h"
#include "more_lowrank.h"
#include "more_pack.h"

namespace more {

struct StreamArgs {
  LowRankArgs base;   // X, N, h, NT (even here), k, packed weights, outputs
  int NB;             // token blocks of 32
  int G;              // waves in the grid (each owns blocks gw, gw + G, ...)
  int KSP;            // K-steps of the down-projection, padded to a multiple of D
};

template <int KMAX, bool FULL, int R16, int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void stream_kernel(StreamArgs sa) {
  const LowRankArgs& a = sa.base;
  constexpr int CAP = Cap<KMAX>::value;
  constexpr int RB = (R16 + 1) / 2;
  extern __shared__ float2 smem_log[];
  const int lane = threadIdx.x & 63;
  // wave-uniform values live in scalar registers, so every branch on the
  // block schedule is a scalar branch and no load ends up under exec masking
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool hi = lane >= 32;
  const int hf = hi ? 1 : 0, col = lane & 31;
  const int gw = blockIdx.x * WAVES + wave;
  if (gw >= sa.NB) return;                                   // wave-uniform
  const int nbw = (sa.NB - gw + sa.G - 1) / sa.G;            // blocks owned by this wave
  LogRef lg{smem_log + (size_t)wave * CAP * kWave};
  const uint16_t* X = (const uint16_t*)a.X;
  const bf16x8* r1p = (const bf16x8*)a.R1p;
  const bf16x8* r2p = (const bf16x8*)a.R2p;
  const uint32_t* bq = a.biasq;
  const int KS = (a.h + 15) / 16;
  const int NBATCH = sa.KSP / D;
  const int NTe = a.NT;                                      // even
  const int NT2 = NTe / 2;

  // ---------------------------------------------------------------- X ring
  auto xaddr = [&](int i, int s) -> const bf16x8* {
    long long row = (long long)(gw + (long long)i * sa.G) * kTile + col;
    row = row < a.N ? row : a.N - 1;
    const int c = (16 * s + 8 * hf < a.h) ? 16 * s + 8 * hf : 16 * s;
    const bool real = (i < nbw) && (s < KS);
    return real ? (const bf16x8*)(X + (size_t)row * a.h + c) : (const bf16x8*)X;
  };
  bf16x8 xr[D], rr[D][RB];
  auto load_slot = [&](bf16x8& xs, bf16x8 (&rs)[RB], int i, int s) {
    xs = __builtin_nontemporal_load(xaddr(i, s));
#pragma unroll
    for (int b = 0; b < RB; ++b) rs[b] = r1p[((size_t)s * RB + b) * kWave + lane];
  };

  // ------------------------------------------------------- sweep operands
  struct Ops {
    bf16x8 w[R16];
    uint32_t b;
  };
  auto load_ops = [&](int t, Ops& o) {
#pragma unroll
    for (int m = 0; m < R16; ++m) o.w[m] = r2p[((size_t)t * R16 + m) * kWave + lane];
    o.b = bq[(size_t)t * kWave + lane];
  };
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)((!hi && e < 2) ? 1.f : 0.f);
  bf16x8 zh[R16], zl[R16];
  auto logits = [&](const Ops& o) {
    bf16x8 ab;
#pragma unroll
    for (int e = 0; e < 8; ++e) ab[e] = (bf16)0.f;
    ab[0] = __builtin_bit_cast(bf16, (uint16_t)(o.b & 0xffffu));
    ab[1] = __builtin_bit_cast(bf16, (uint16_t)(o.b >> 16));
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

  floatx16 zacc[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) zacc[b][v] = 0.f;
#pragma unroll
  for (int m = 0; m < R16; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      zh[m][e] = (bf16)0.f;
      zl[m][e] = (bf16)0.f;
    }

  // prologue: the first D K-steps of block 0, the first two tiles' operands
#pragma unroll
  for (int u = 0; u < D; ++u) load_slot(xr[u], rr[u], 0, u);
  Ops o0, o1;
  load_ops(0, o0);
  load_ops(1, o1);
  SweepState<KMAX, CAP> st;
  floatx16 accA;

  // i = -1 only streams block 0; i = nbw - 1 only sweeps the last block.
  for (int i = -1; i < nbw; ++i) {
    const bool has_cur = i >= 0, has_nxt = i + 1 < nbw;
    if (has_cur) {
      st.init(a.k);
      accA = logits(o0);                    // tile 0 (o0 holds its operands)
    }
    load_ops(has_cur ? 2 % NTe : 0, o0);    // tile 2 next; before block 0 keep tile 0
    for (int j = 0; j < NBATCH; ++j) {
      // refill targets: K-step s + D of block i+1, or the first K-steps of block i+2
      const bool wrap = j + 1 >= NBATCH;
      const int ib = wrap ? i + 2 : i + 1;
#pragma unroll
      for (int u = 0; u < D; ++u) {
        if (has_nxt) {
#pragma unroll
          for (int b = 0; b < RB; ++b) zacc[b] = mfma_bf16(rr[u][b], xr[u], zacc[b]);
        }
        const int sb = wrap ? u : (j + 1) * D + u;
        load_slot(xr[u], rr[u], ib, sb);
      }
      if (has_cur) {
        const int p0 = j * NT2 / NBATCH, p1 = (j + 1) * NT2 / NBATCH;
        for (int p = p0; p < p1; ++p) {
          const int t = 2 * p;
          floatx16 accB = logits(o1);       // tile t+1
          load_ops((t + 3) % NTe, o1);
          st.template tile<FULL>(accA, kTile * t + 4 * hf, lg, lane, hi, a.perm, a.k);
          accA = logits(o0);                // tile t+2 (unused after the last pair)
          load_ops(p == NT2 - 1 ? 0 : (t + 4) % NTe, o0);
          st.template tile<FULL>(accB, kTile * (t + 1) + 4 * hf, lg, lane, hi, a.perm, a.k);
        }
      }
    }
    if (has_cur) {
      const long long n = (long long)(gw + (long long)i * sa.G) * kTile + col;
      finish_tokens<KMAX, CAP, FULL>(st, lg, lane, hi, n < a.N, n, a.perm, a.k, a.out_idx,
                                     a.out_gate, a.out_logit, a.out_lse);
    }
    if (has_nxt) {
#pragma unroll
      for (int m = 0; m < R16; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = zacc[m >> 1][8 * (m & 1) + e];
          const bf16 hv = (bf16)f;
          zh[m][e] = hv;
          zl[m][e] = (bf16)(f - (float)hv);
        }
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) zacc[b][v] = 0.f;
    }
  }
}

}  // namespace more
