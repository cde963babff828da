// more_splitm.h -- the low-rank router for few tokens and many experts
// (decode): the expert range is split over many waves.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.1 Algorithm 1 (z = X-block times the down-projection, then
// a sweep over the experts with a running top-k) and App. E.3 (a top-k over
// shards of the experts, merged; the full-softmax normaliser combined across
// shards by eq. (8)).
//
// With N = 256 tokens there are 8 blocks of 32: one wave per block leaves
// almost the whole GPU idle while each wave sweeps M = 65536 experts.  Here
//   splitm_proj_kernel   wave (block, K-part): z of the block over an eighth
//                        of the hidden units (fp32 partial sums);
//   splitm_route_kernel  wave (block, shard): z = the sum of the partials, in
//                        a fixed order; then the exact two-half sweep of
//                        more_lowrank.h over the shard's expert tiles only,
//                        finished as the shard's k best (logit, expert) and
//                        its log-sum-exp;
//   merge_kernel         (more_merge.h) the k best of the shards' lists, and
//                        the gates.
// Shards are ranges of sweep tiles (at least 4 tiles each, so every shard
// holds a real expert); the candidates carry global expert indices.
#pragma once
#include "more_device.h"
#include "more_lowrank.h"
#include "more_twopass.h"

namespace more {

constexpr int kSplitmKParts = 8;   // K-parts of the projection

struct SplitmProjArgs {
  const void* X;
  long long N;
  int h;
  int NB;            // 32-token blocks
  int KS;            // 16-column K-steps of h
  int KPS;           // K-steps per part
  const void* R1p;   // packed down-projection (A operands of the 32x32x16 MFMA)
  float* part;       // [kSplitmKParts][NB][RB][16][64 lanes] fp32
};

// one wave per workgroup (spread over the CUs): block b = wg / kSplitmKParts,
// part p = wg % kSplitmKParts
template <int R16>
__global__ __launch_bounds__(64) void splitm_proj_kernel(SplitmProjArgs a) {
  constexpr int RB = (R16 + 1) / 2;
  const int lane = threadIdx.x;
  const int b = blockIdx.x / kSplitmKParts, p = blockIdx.x % kSplitmKParts;
  const bool hi = lane >= 32;
  const int hf = hi ? 1 : 0, col = lane & 31;
  const long long n = (long long)b * kTile + col;
  const long long row = n < a.N ? n : a.N - 1;
  const uint16_t* xrow = (const uint16_t*)a.X + (size_t)row * a.h;
  const bf16x8* r1p = (const bf16x8*)a.R1p;
  floatx16 z[RB];
#pragma unroll
  for (int q = 0; q < RB; ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) z[q][v] = 0.f;
  const int s0 = p * a.KPS, s1 = min(s0 + a.KPS, a.KS);
  // groups of 4 K-steps, the next group's loads in flight while one is
  // multiplied (clamped K-steps past the part re-read its last one; their
  // products are skipped)
  constexpr int U = 4;
  auto xaddr = [&](int s) {
    const int c = (16 * s + 8 * hf < a.h) ? 16 * s + 8 * hf : 16 * s;   // a half-filled last K-step
    return (const bf16x8*)(xrow + c);
  };
  auto load = [&](int s, bf16x8 (&xs)[U], bf16x8 (&rs)[U][RB]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sc = min(s + u, s1 - 1);
      xs[u] = __builtin_nontemporal_load(xaddr(sc));
#pragma unroll
      for (int q = 0; q < RB; ++q) rs[u][q] = r1p[((size_t)sc * RB + q) * kWave + lane];
    }
  };
  auto compute = [&](int s, const bf16x8 (&xs)[U], const bf16x8 (&rs)[U][RB]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s + u < s1) {
#pragma unroll
        for (int q = 0; q < RB; ++q) z[q] = mfma_bf16(rs[u][q], xs[u], z[q]);
      }
  };
  if (s0 < s1) {
    bf16x8 xa[U], ra[U][RB], xb[U], rb[U][RB];
    load(s0, xa, ra);
    int s = s0;
    for (; s + U < s1; s += 2 * U) {
      load(s + U, xb, rb);
      compute(s, xa, ra);
      load(min(s + 2 * U, s1 - 1), xa, ra);
      compute(s + U, xb, rb);
    }
    if (s < s1) compute(s, xa, ra);
  }
  float* dst = a.part + ((size_t)p * a.NB + b) * RB * 16 * kWave;
#pragma unroll
  for (int q = 0; q < RB; ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) dst[((size_t)q * 16 + v) * kWave + lane] = z[q][v];
}

// The routing kernel's selection for a shard: the two-pass group log of
// more_twopass.h where its per-wave LDS (log of KMAX + 2 groups per lane,
// result block) fits four waves in a workgroup, the running top-k above.
template <int KMAX>
struct SplitmTwoPass {
  static constexpr bool value = KMAX <= 16;
  static constexpr int kCapG = KMAX + 2;
  static constexpr int kValBytes = kCapG * kWave * 16;
  static constexpr int kPosBytes = kCapG * kWave * 4;
  static constexpr int kWaveBytes = kValBytes + kPosBytes + TpStage<KMAX>::kWords * 4;
};

// Dynamic LDS of splitm_route_kernel (four waves).
inline size_t splitm_lds_bytes(int kmax) {
  switch (kmax) {
    case 4: return 4 * (size_t)SplitmTwoPass<4>::kWaveBytes;
    case 8: return 4 * (size_t)SplitmTwoPass<8>::kWaveBytes;
    case 16: return 4 * (size_t)SplitmTwoPass<16>::kWaveBytes;
    default: return 4 * (size_t)(2 * kmax + 8) * kWave * sizeof(float2);   // running top-k log
  }
}

struct SplitmArgs {
  LowRankArgs base;     // N, NT, k, R2p, biasq, perm (outputs unused)
  const float* part;    // from splitm_proj_kernel
  int NB;               // 32-token blocks
  int TPS;              // tiles per shard (>= 4; the last shard may be shorter)
  int S;                // shards
  float* cand_logit;    // [S][N][k]
  int* cand_idx;        // [S][N][k] global expert indices
  float* cand_gate;     // [S][N][k] scratch (the per-shard gates are not used)
  float* shard_lse;     // [S][N] (full-softmax gate) or null
};

// wave (block b, shard s) = global wave index s * NB + b (the blocks of one
// shard are neighbours: they share the shard's R2 tiles in L2)
template <int KMAX, bool FULL, int R16>
__global__ __launch_bounds__(256) void splitm_route_kernel(SplitmArgs sa) {
  const LowRankArgs& a = sa.base;
  constexpr int CAP = Cap<KMAX>::value;
  constexpr int RB = (R16 + 1) / 2;
  extern __shared__ float2 smem_log[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gw = blockIdx.x * 4 + wave;
  if (gw >= sa.NB * sa.S) return;   // wave-uniform
  const int s = gw / sa.NB, b = gw % sa.NB;
  const bool hi = lane >= 32;
  const int hf = hi ? 1 : 0, col = lane & 31;
  const long long n = (long long)b * kTile + col;
  const bool rowok = n < a.N;
  LogRef lg{smem_log + (size_t)wave * CAP * kWave};

  // z of the block: the K-parts summed in a fixed order
  floatx16 z[RB];
#pragma unroll
  for (int q = 0; q < RB; ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) z[q][v] = 0.f;
  for (int p = 0; p < kSplitmKParts; ++p) {
    const float* src = sa.part + ((size_t)p * sa.NB + b) * RB * 16 * kWave;
#pragma unroll
    for (int q = 0; q < RB; ++q)
#pragma unroll
      for (int v = 0; v < 16; ++v) z[q][v] += src[((size_t)q * 16 + v) * kWave + lane];
  }
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
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)((!hi && e < 2) ? 1.f : 0.f);
  const bf16x8* r2p = (const bf16x8*)a.R2p;
  const uint32_t* bq = a.biasq;
  const int t0 = s * sa.TPS, t1 = min(t0 + sa.TPS, a.NT);
  struct Ops {
    bf16x8 w[R16];
    uint32_t b;
  };
  auto load_ops = [&](int t, Ops& o) {
    const int tc = t < t1 ? t : t1 - 1;   // clamped: always a tile of the shard
#pragma unroll
    for (int m = 0; m < R16; ++m) o.w[m] = r2p[((size_t)tc * R16 + m) * kWave + lane];
    o.b = bq[(size_t)tc * kWave + lane];
  };
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
  // the shard's tiles with two in flight, as in lowrank_kernel; on_tile(acc, t)
  auto sweep = [&](auto&& on_tile) {
    Ops o0, o1;
    load_ops(t0, o0);
    load_ops(t0 + 1, o1);
    floatx16 accA = logits(o0);
    load_ops(t0 + 2, o0);
    for (int t = t0; t < t1; t += 2) {
      floatx16 accB = logits(o1);
      load_ops(t + 3, o1);
      on_tile(accA, t);
      accA = logits(o0);   // beyond the shard's last tile: unused
      load_ops(t + 4, o0);
      if (t + 1 < t1) on_tile(accB, t + 1);
    }
  };
  const size_t so = (size_t)s * a.N;
  if constexpr (SplitmTwoPass<KMAX>::value) {
    // Two passes over the shard (more_twopass.h): the 4-logit group maxima give
    // a lower bound of each token's k-th logit, the second pass logs the 4-logit
    // groups that reach it (and accumulates eq. 8), and one ordered finish
    // forms the shard's k best.  Wave-wide work per tile stays small: a
    // running top-k would insert a logit whenever any of the 64 lanes holds
    // one above its own k-th.
    typedef SplitmTwoPass<KMAX> TP;
    typedef TpStage<KMAX> SG;
    char* wl = (char*)smem_log + (size_t)wave * TP::kWaveBytes;
    const GroupLog glog{(lds_f4*)wl, (lds_i32*)(wl + TP::kValBytes)};
    lds_f32* stg = (lds_f32*)(wl + TP::kValBytes + TP::kPosBytes);
    TwoPassState<KMAX> st;
    st.init(a.k);
    sweep([&](const floatx16& acc, int) { tp_pass1_groups<KMAX>(st, acc); });
    tp_threshold<KMAX>(st, hi, a.k);
    sweep([&](const floatx16& acc, int t) {
      const floatx4 g = tp_pass2_scan<KMAX, false>(st, acc, false);
      if (FULL) tp_lse_tile<KMAX>(st, acc, g);
      tp_pass2_groups<KMAX, TP::kCapG>(st, acc, g, kTile * t + 4 * hf, glog, lane, a.perm, a.k);
    });
    tp_finish_groups<KMAX, false, FULL>(st, glog, lane, hi, a.perm, a.k, true, stg);
    lds_drain();
    // the block's rows of the stage (token t's k entries at t k .. t k + k - 1)
    // -> the shard's candidate lists; rows past N are dropped
    const long long n0 = (long long)b * kTile;
    const int rows = a.N - n0 < kTile ? (int)(a.N - n0) : kTile;
    const int words = rows * a.k;
    int* ci = sa.cand_idx + (so + n0) * a.k;
    float* cl = sa.cand_logit + (so + n0) * a.k;
    for (int c = lane; c < words; c += kWave) {
      ci[c] = __float_as_int(stg[SG::kIdx + c]);
      cl[c] = stg[SG::kLogit + c];
    }
    if (FULL && lane < rows) sa.shard_lse[so + n0 + lane] = stg[SG::kLse + lane];
  } else {
    SweepState<KMAX, CAP> st;
    st.init(a.k);
    sweep([&](const floatx16& acc, int t) {
      st.template tile<FULL>(acc, kTile * t + 4 * hf, lg, lane, hi, a.perm, a.k);
    });
    finish_tokens<KMAX, CAP, FULL, true>(st, lg, lane, hi, rowok, n, a.perm, a.k, sa.cand_idx + so * a.k,
                                   sa.cand_gate + so * a.k, sa.cand_logit + so * a.k,
                                   FULL ? sa.shard_lse + so : nullptr);
  }
}

}  // namespace more
