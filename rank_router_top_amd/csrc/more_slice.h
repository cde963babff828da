// more_slice.h -- expert-slice form of the fused low-rank router for gfx950
// (bf16 storage, r in {16, 32}, M = 4096 experts, k <= 8).
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.1 Algorithm 1: per block of tokens, z = X-block times the
// down-projection stays on chip, the experts are swept tile by tile and only
// the top-k (value, index) pairs and gates reach HBM (Fig. 12 gates; App.
// F.2.1 eq. (6)/(8) for the full-softmax probability).
//
// Why this form.  The up-projection R2 (r x M bf16, 256 KiB at r = 32) is
// read by every token block.  Streaming it from L2 for each 32-token block
// moves four times the bytes of X through each CU's vector-memory path, and
// that path is also the one the X stream needs.  Here R2 never moves after
// the start: the 8 consumer waves of a workgroup each own a fixed slice of
// 16 expert tiles (local tile i = global tile c + 8i, so the bias-sorted
// sweep order spreads the high-bias tiles over all waves), TV of them in
// VGPRs and the rest in LDS.  All 8 consumers work on the same token block;
// 4 producer waves (more_pc.h) stream X and hand over z through a 2- or
// 3-slot LDS ring.
//
// Exact top-k with a per-block threshold (every step keeps the exact result):
//   pass 1: hi-only logits s~ = (R2 tile)^T z_hi, no bias: per lane-half and
//     tile, LB = max(s~) + min(bias of the tile) is at most the approximate
//     logit of one real expert.  Each lane-half keeps its two largest LB.
//   exchange (consumer barrier): thr = k-th largest of the 32 values of the
//     token (16 lane-halves x 2).  With eps bounding |exact - approx|, at least
//     k experts have an exact logit >= thr - eps, so the token's k-th logit is
//     >= thr - eps.
//   pass 2: s~ again; a tile is worked on only if max(s~) + max(bias of the
//     tile) >= thr - 2 eps in some lane (a necessary condition for holding a
//     top-k logit).  Active tiles are recomputed exactly (bias as the MFMA
//     accumulator input, z as bf16 hi + lo) and every logit >= thr - eps is
//     appended with its expert index to the token's log in LDS.
//   finish (consumer barrier): wave c ranks the logged candidates of tokens
//     4c .. 4c+3 by (logit desc, expert index asc), computes the gates and
//     stores them.
// eps = ||z_lo|| * max_m ||R2[:, m]|| (the dropped z_lo term, Cauchy-Schwarz)
// plus 2^-16 (||z_hi|| max_m ||R2[:, m]|| + max |b|), which bounds the fp32
// accumulation differences of the two MFMA chains.  In the full-softmax mode
// pass 1 uses exact logits, which also feed the running maximum and
// normaliser of eq. (8).
//
// A token whose log overflows (massive exact ties, adversarial inputs) is
// routed again by its finishing wave on a slow exact path: every tile of the
// token recomputed with the same MFMA chain (operands from global memory) and
// a per-lane ordered top-k.  No other wave takes part.
#pragma once
#include "more_pc.h"
#include "more_twopass.h"

namespace more {

constexpr int kSlCons = 8;                    // consumer waves
constexpr int kSlWaves = kPcProd + kSlCons;   // 12 waves: 3 per SIMD
constexpr int kSlTPW = 16;                    // expert tiles per consumer
constexpr int kSlNT = kSlCons * kSlTPW;       // 128 tiles: M = 4096
constexpr int kSlCap = 32;                    // log entries per token and block
constexpr int kSlK = 8;                       // largest k

// LDS flag words (ints)
constexpr int kSlFull = 0;    // [kSlNZ] last block published in each z slot, +1
constexpr int kSlBar0 = 4;    // consumer barrier counters
constexpr int kSlBar1 = 5;    // also tells producers that a z slot may be reused
constexpr int kSlBar2 = 6;
constexpr int kSlAbort = 8;
constexpr int kSlZOff = 1536;   // LDS: flags, statistics, counters, bias bounds, then the z ring
constexpr int kSlLogStride = kSlCap + 2;   // entries per token log: CAP, the spare slot, padding to 16 B

struct SlArgs {
  LowRankArgs base;   // X, N, h, k, R2p / biasp / perm in sweep order, outputs
  const void* R1q;    // producer A operands (more_pc.h)
  int NB;             // 32-token blocks
  int G;              // workgroups
  int KSP;            // producer K-steps
  int spin_limit;     // polls before a wait gives up
};

// LDS map (bytes); NZ z-ring slots
template <bool FULL, bool BIAS, int R16, int TV, int NZ>
struct SlLds {
  static constexpr int TL = kSlTPW - TV;                        // tiles kept in LDS
  static constexpr int kStat = 64;                              // [cons] (max ||R2 col||^2, max |b|)
  static constexpr int kCnt = 128;                              // [2][32] int: log counts (block parity)
  static constexpr int kBmm = 512;                              // [cons][16] (min, max) bias of a tile
  static constexpr int kZ = kSlZOff;                            // [NZ][hi, lo][R16][64][16 B]
  static constexpr int kR2 = kZ + NZ * 2 * R16 * 1024;          // [cons][TL][R16][64][16 B]
  static constexpr int kBias = kR2 + kSlCons * TL * R16 * 1024; // [NT][2][16] f32
  static constexpr int kPerm = kBias + (BIAS ? kSlNT * 128 : 0);   // [NT*32] u16 expert of a position
  static constexpr int kLog = kPerm + kSlNT * 64;               // [32][kSlLogStride] (logit, position / expert)
  static constexpr int kExch = kLog + 32 * kSlLogStride * 8;    // [32][16 lane halves] 2 x f32
  static constexpr int kMZ = kExch + 32 * 16 * 8;               // FULL: [2][32][16] (m, Z)
  static constexpr int kStage = kMZ + (FULL ? 2 * 32 * 16 * 8 : 0);   // [32][kSlK] (expert, gate)
  static constexpr int bytes = kStage + 32 * kSlK * 8;
};

// Producer side of the ring: block i goes to slot i % NZ once every consumer
// has finished block i - NZ (finish included: its slow path reads z from the
// slot), i.e. has arrived at the first barrier of the next block.
template <int R16, int NZ>
struct SlHandOff {
  char* lds;
  int limit;
  __device__ __forceinline__ char* acquire(int i) const {
    flag_ptr fl = pc_flags(lds);
    if (i >= NZ && !pc_wait(fl + kSlBar1, kSlCons * (i - NZ + 2), fl + kSlAbort, limit)) return nullptr;
    return lds + kSlZOff + (i % NZ) * 2 * R16 * 1024;
  }
  __device__ __forceinline__ void publish(int i) const {
    lds_drain();
    pc_flags(lds)[kSlFull + i % NZ] = i + 1;
  }
  __device__ __forceinline__ bool retire(int, int) const { return true; }   // consumers store their own results
  __device__ __forceinline__ void finish(int, int) const {}
};

// Barrier of the 8 consumer waves: arrive (release), then wait for `target`
// arrivals.  Bounded like every wait of the kernel.
__device__ __forceinline__ bool sl_bar(flag_ptr ctr, int target, flag_ptr abort_word, int limit, int lane) {
  if (lane == 0) __hip_atomic_fetch_add((lds_i32*)ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  return pc_wait(ctr, target, abort_word, limit);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
// Sum / max over the 16 lanes of a row (lanes 16t .. 16t+15).
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float bf16_sq_sum(const bf16x8& v) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = (float)v[e];
    s = __builtin_fmaf(f, f, s);
  }
  return s;
}

// (a, ia) ranks before (b, ib): larger logit, then lower expert index.
__device__ __forceinline__ bool beats(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// Slow exact path for tokens whose log overflowed (bits of tok_mask: token
// columns of the block).  The whole wave recomputes every tile with the same
// MFMA chain as the fast path (bias as the accumulator input, z hi then lo),
// reading the operands from global memory; lane l keeps an ordered top-k of
// its column's half-tile rows, the two halves are merged, and the lanes of
// the masked columns store the result.  App. F.1 Algorithm 1 in its plain
// form (one running top-k per token over all experts).
template <bool FULL, bool BIAS, int R16>
__device__ __forceinline__ void sl_slow(const LowRankArgs& a, const char* zs, int2* stage, int lane,
                                       uint32_t tok_mask, long long n0) {
  const int hf = lane >> 5, tl = lane & 31;
  bf16x8 zh[R16], zl[R16];
#pragma unroll
  for (int m = 0; m < R16; ++m) {
    zh[m] = *(const bf16x8*)(zs + m * 1024 + lane * 16);
    zl[m] = *(const bf16x8*)(zs + (R16 + m) * 1024 + lane * 16);
  }
  const bool hi = hf != 0;
  const int k = a.k;
  const rsrc_t r2d = make_rsrc(a.R2p, kSlNT * R16 * 1024);
  float V[kSlK];
  int IX[kSlK];
#pragma unroll
  for (int j = 0; j < kSlK; ++j) {
    V[j] = -__builtin_inff();
    IX[j] = 0x7fffffff;
  }
  float m = kLowest * 0.25f, Z = 0.f;
  for (int t = 0; t < kSlNT; ++t) {
    floatx16 acc = {};
    if constexpr (BIAS) acc = *(const floatx16*)(a.biasp + (2 * t + hf) * 16);
    bf16x8 w[R16];
#pragma unroll
    for (int mm = 0; mm < R16; ++mm) w[mm] = buf_load(r2d, lane * 16 + mm * 1024, t * R16 * 1024);
#pragma unroll
    for (int mm = 0; mm < R16; ++mm) acc = mfma_bf16(w[mm], zh[mm], acc);
#pragma unroll
    for (int mm = 0; mm < R16; ++mm) acc = mfma_bf16(w[mm], zl[mm], acc);
    if constexpr (FULL) {
      const float mn = fmaxf(m, max16(acc));
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) s += __builtin_amdgcn_exp2f((acc[v] - mn) * kLog2e);
      Z = Z * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + s;
      m = mn;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float x = acc[v];
      if (x >= V[kSlK - 1]) {
        const int pos = kTile * t + 8 * (v >> 2) + 4 * hf + (v & 3);
        ordered_insert<kSlK>(V, IX, x, a.perm[pos]);
      }
    }
  }
  // merge the two halves of each token (the low lane ends up with the result)
#pragma unroll
  for (int j = 0; j < kSlK; ++j) {
    const float pv = partner_f32(V[j], hi);
    const int pi = (int)partner_u32((uint32_t)IX[j], hi);
    if (!hi) ordered_insert<kSlK>(V, IX, pv, pi);
  }
  float lse = 0.f;
  if constexpr (FULL) {
    const float mp = partner_f32(m, hi), Zp = partner_f32(Z, hi);
    const float mm = fmaxf(m, mp);
    lse = mm + __builtin_amdgcn_logf(Z * __builtin_amdgcn_exp2f((m - mm) * kLog2e) +
                                     Zp * __builtin_amdgcn_exp2f((mp - mm) * kLog2e)) * kLn2;
  }
  const long long n = n0 + tl;
  if (hi || !((tok_mask >> tl) & 1) || n >= a.N) return;
  // FULL: eq. (6) at the selected experts; otherwise Fig. 12 (max subtracted)
  const float ref = FULL ? lse : V[0];
  float w[kSlK];
  float den = 0.f;
#pragma unroll
  for (int j = 0; j < kSlK; ++j) {
    w[j] = (j < k) ? __builtin_amdgcn_exp2f((V[j] - ref) * kLog2e) : 0.f;
    den += w[j];
  }
  const float inv = FULL ? 1.f : 1.f / den;
  const size_t o = (size_t)n * k;
#pragma unroll
  for (int j = 0; j < kSlK; ++j) {
    if (j < k) {
      stage[tl * kSlK + j] = make_int2(IX[j], __float_as_int(w[j] * inv));
      if (a.out_logit) a.out_logit[o + j] = V[j];
    }
  }
  if (FULL && a.out_lse) a.out_lse[n] = lse;
}

template <bool FULL, bool BIAS, int R16, int TV, int NZ>
__device__ __forceinline__ void sl_consume(const SlArgs& sa, char* lds, int c, int lane, int nbw) {
  typedef SlLds<FULL, BIAS, R16, TV, NZ> L;
  constexpr int TL = L::TL;
  constexpr int CAP = kSlCap;
  const LowRankArgs& a = sa.base;
  const int k = a.k;
  flag_ptr fl = pc_flags(lds);
  flag_ptr abort_word = fl + kSlAbort;
  const int limit = sa.spin_limit;
  const int hf = lane >> 5, tl = lane & 31;
  const bool hi = hf != 0;
  lds_i32* cnt_all = (lds_i32*)(lds + L::kCnt);

  // ---- stationary operands: R2^T tiles of this consumer's slice
  const rsrc_t r2d = make_rsrc(a.R2p, kSlNT * R16 * 1024);
  bf16x8 A[TV][R16];
  float cn2 = 0.f;   // largest squared column norm of R2 in the slice
#pragma unroll
  for (int i = 0; i < TV; ++i) {
    float s = 0.f;
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      A[i][m] = buf_load(r2d, lane * 16 + m * 1024, (c + 8 * i) * R16 * 1024);
      s += bf16_sq_sum(A[i][m]);
    }
    cn2 = fmaxf(cn2, s + partner_f32(s, hi));
  }
  char* my_r2 = lds + L::kR2 + c * TL * R16 * 1024;
#pragma unroll
  for (int i = 0; i < TL; ++i) {
    float s = 0.f;
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      const bf16x8 w = buf_load(r2d, lane * 16 + m * 1024, (c + 8 * (TV + i)) * R16 * 1024);
      *(bf16x8*)(my_r2 + (i * R16 + m) * 1024 + lane * 16) = w;
      s += bf16_sq_sum(w);
    }
    cn2 = fmaxf(cn2, s + partner_f32(s, hi));
  }
  auto tileA = [&](int i, int m) -> bf16x8 {
    if (i < TV) return A[i < TV ? i : 0][m];
    return *(const bf16x8*)(my_r2 + ((i - TV) * R16 + m) * 1024 + lane * 16);
  };
  auto bias_tile = [&](int i) -> floatx16 {
    return *(const floatx16*)(lds + L::kBias + (2 * (c + 8 * i) + hf) * 64);
  };

  // ---- bias range of every local tile (wave-uniform), and the global bounds
  float2* bmm = (float2*)(lds + L::kBmm) + c * kSlTPW;
  float babs = 0.f;
#pragma unroll
  for (int i = 0; i < kSlTPW; ++i) {
    if constexpr (BIAS) {
      const floatx16 b = bias_tile(i);
      float lo = b[0], up = b[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) {
        lo = fminf(lo, b[v]);
        up = fmaxf(up, b[v]);
      }
      lo = fminf(lo, partner_f32(lo, hi));
      up = fmaxf(up, partner_f32(up, hi));
      if (lane == 0) bmm[i] = make_float2(lo, up);
      babs = fmaxf(babs, fmaxf(fabsf(lo), fabsf(up)));
    } else {
      if (lane == 0) bmm[i] = make_float2(0.f, 0.f);
    }
  }
  cn2 = wave_max(cn2);
  if (lane == 0) *(float2*)(lds + L::kStat + 8 * c) = make_float2(cn2, babs);
  if (!sl_bar(fl + kSlBar0, kSlCons, abort_word, limit, lane)) return;
  float cmax2 = 0.f, bmax_abs = 0.f;
#pragma unroll
  for (int w = 0; w < kSlCons; ++w) {
    const float2 st = *(const float2*)(lds + L::kStat + 8 * w);
    cmax2 = fmaxf(cmax2, st.x);
    bmax_abs = fmaxf(bmax_abs, st.y);
  }
  const float cmax = __builtin_sqrtf(cmax2) * (1.f + 0x1p-16f);   // covers the fp32 sums and the root

  // Results leave through a staging area: the finish of block j puts this
  // wave's (expert, gate) pairs there, and the same wave stores them during
  // block j + 1, right after the first tile of pass 2.  The consumer issues no
  // other global memory operation in the loop, so those stores can take as
  // long as writes take under the X stream without any wait of the wave on
  // them (a vector-memory wait would also wait for every earlier store).
  int2* stage = (int2*)(lds + L::kStage);
  auto copy_out = [&](int jb) {
    // tokens 4c .. 4c+3 of block jb: lane -> token 4c + lane/16, ranks 2(lane%16) .. +1
    const int t = 4 * c + (lane >> 4), r = 2 * (lane & 15);
    const long long n = ((long long)blockIdx.x + (long long)jb * sa.G) * kTile + t;
    if (r < k && n < a.N) {
      const int4 v = *(const int4*)(stage + t * kSlK + r);   // pairs r, r + 1
      const size_t o = (size_t)n * k + r;
      a.out_idx[o] = v.x;
      a.out_gate[o] = __int_as_float(v.y);
      if (r + 1 < k) {
        a.out_idx[o + 1] = v.z;
        a.out_gate[o + 1] = __int_as_float(v.w);
      }
    }
  };
  for (int jj = 0; jj < nbw; ++jj) {
    const int slot = jj % NZ;
    if (!pc_wait(fl + kSlFull + slot, jj + 1, abort_word, limit)) return;
    const char* zs = lds + L::kZ + slot * 2 * R16 * 1024;
    // z_hi stays in registers for the block; z_lo is read from the slot where
    // it is needed (exact tiles), the slot stays valid until the block is done
    bf16x8 zh[R16];
#pragma unroll
    for (int m = 0; m < R16; ++m) zh[m] = *(const bf16x8*)(zs + m * 1024 + lane * 16);
    auto zlo = [&](int m) -> bf16x8 { return *(const bf16x8*)(zs + (R16 + m) * 1024 + lane * 16); };
    // eps: bound on |exact logit - (approximate logit + bias)| for this token
    float nh = 0.f, nl = 0.f;
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      nh += bf16_sq_sum(zh[m]);
      nl += bf16_sq_sum(zlo(m));
    }
    nh += partner_f32(nh, hi);
    nl += partner_f32(nl, hi);
    const float eps = __builtin_sqrtf(nl) * cmax * (1.f + 0x1p-10f) +
                      0x1p-16f * (__builtin_sqrtf(nh) * cmax + bmax_abs);
    const int par = jj & 1;

    auto approx = [&](int i) -> floatx16 {
      floatx16 acc = {};
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(tileA(i, m), zh[m], acc);
      return acc;
    };
    auto exact = [&](int i) -> floatx16 {
      floatx16 acc = {};
      if constexpr (BIAS) acc = bias_tile(i);
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(tileA(i, m), zh[m], acc);
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(tileA(i, m), zlo(m), acc);
      return acc;
    };

    // ---- pass 1: two largest tile bounds per lane-half (FULL: exact logits,
    // running maximum and normaliser of eq. 8)
    float t0 = kLowest, t1 = kLowest;
    float m1 = kLowest * 0.25f, Z1 = 0.f;
#pragma unroll
    for (int i = 0; i < kSlTPW; ++i) {
      const floatx16 acc = FULL ? exact(i) : approx(i);
      const float tm = max16(acc);
      const float lb = (BIAS && !FULL) ? tm + bmm[i].x : tm;   // FULL: exact logits, bias included
      t1 = __builtin_amdgcn_fmed3f(t0, t1, lb);
      t0 = fmaxf(t0, lb);
      __builtin_amdgcn_sched_barrier(0);   // one tile at a time (register pressure)
      if constexpr (FULL) {
        const float mn = fmaxf(m1, tm);
        const float mb = mn * kLog2e;
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) s += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], kLog2e, -mb));
        Z1 = Z1 * __builtin_amdgcn_exp2f((m1 - mn) * kLog2e) + s;
        m1 = mn;
      }
    }
    *(float2*)(lds + L::kExch + (tl * 16 + 2 * c + hf) * 8) = make_float2(t0, t1);
    if constexpr (FULL) *(float2*)(lds + L::kMZ + ((par * 32 + tl) * 16 + 2 * c + hf) * 8) = make_float2(m1, Z1);
    if (!sl_bar(fl + kSlBar1, kSlCons * (jj + 1), abort_word, limit, lane)) return;
    // every wave has finished the previous block: clear this wave's tokens'
    // counters of the next block (same parity as the previous one)
    if (lane < 4) cnt_all[(par ^ 1) * 32 + 4 * c + lane] = 0;

    // ---- threshold: k-th largest of the token's 32 bounds (both lanes agree)
    float thr;
    {
      float T[kSlK];
#pragma unroll
      for (int j = 0; j < kSlK; ++j) T[j] = (j < kSlK - k) ? __builtin_inff() : kLowest;
      const float4* ex = (const float4*)(lds + L::kExch + (tl * 16 + 8 * hf) * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = ex[q];
        med3_insert<kSlK>(T, v.x);
        med3_insert<kSlK>(T, v.y);
        med3_insert<kSlK>(T, v.z);
        med3_insert<kSlK>(T, v.w);
      }
      float U[kSlK];
#pragma unroll
      for (int j = 0; j < kSlK; ++j) U[j] = T[j];
#pragma unroll
      for (int j = 0; j < kSlK; ++j) {
        const float p = partner_f32(T[j], hi);
        med3_insert<kSlK>(U, j >= kSlK - k ? p : kLowest);   // the partner's +inf pads are skipped
      }
      thr = U[kSlK - 1];
    }

    // ---- pass 2: append every exact logit >= T1 with its sweep position to
    // the token's log; slots past CAP go to the spare slot CAP (overflow)
    const float T1 = FULL ? thr : thr - eps;   // lower bound of the exact k-th logit
    const float T2 = T1 - eps;                 // the same for approximate logits
    lds_i32* cnt = cnt_all + par * 32;
    float2* lg = (float2*)(lds + L::kLog) + tl * kSlLogStride;
    // sweep position of row 4hf of local tile 0; opaque to the optimiser so that
    // the 256 per-lane positions of the sweep are formed where they are used
    // instead of being hoisted out of the block loop into registers
    int pbase = kTile * c + 4 * hf;
    asm volatile("" : "+v"(pbase));
#pragma unroll
    for (int i = 0; i < kSlTPW; ++i) {
      const floatx16 acc = approx(i);
      float tm = max16(acc);
      if (BIAS) tm += bmm[i].y;
      if (any_lane(tm >= T2)) {
        const floatx16 ex = exact(i);
        const int p0 = pbase + kTile * 8 * i;   // sweep position of row 4hf
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float g = fmaxf(fmaxf(ex[4 * q], ex[4 * q + 1]), fmaxf(ex[4 * q + 2], ex[4 * q + 3]));
          if (any_lane(g >= T1)) {
            bool ok[4];
            int n_ok = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ok[e] = ex[4 * q + e] >= T1;
              n_ok += ok[e] ? 1 : 0;
            }
            // the low lane reserves room for both halves of the token
            const int n_p = (int)partner_u32((uint32_t)n_ok, hi);
            int base = 0;
            if (!hi && n_ok + n_p > 0)
              base = __hip_atomic_fetch_add(cnt + tl, n_ok + n_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            const int pb = (int)partner_u32((uint32_t)base, hi);
            if (hi) base = pb + n_p;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (any_lane(ok[e])) {
                const int slot = ok[e] ? min(base, CAP) : CAP;
                lg[slot] = make_float2(ex[4 * q + e], __int_as_float(p0 + 8 * q + e));
                base += ok[e] ? 1 : 0;
              }
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one tile at a time (register pressure)
      if (i == 0 && jj > 0) {
        copy_out(jj - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!sl_bar(fl + kSlBar2, kSlCons * (jj + 1), abort_word, limit, lane)) return;

    // ---- finish: tokens 4c .. 4c+3 of the block, 16 lanes each
    {
      const int tq = lane >> 4, j16 = lane & 15;
      const int nloc = 4 * c + tq;
      const long long n = ((long long)blockIdx.x + (long long)jj * sa.G) * kTile + nloc;
      float2* lt = (float2*)(lds + L::kLog) + nloc * kSlLogStride;
      const int cn_raw = cnt[nloc];
      const bool ovf = cn_raw > CAP;
      const int cn = ovf ? 0 : cn_raw;
      const bool v0 = j16 < cn, v1 = j16 + 16 < cn;
      // sweep position -> expert, in place (each lane its own two entries)
      float2 e0 = lt[j16], e1 = lt[j16 + 16];
      const unsigned short* pm = (const unsigned short*)(lds + L::kPerm);
      const int i0 = pm[__float_as_int(e0.y) & 0xfff], i1 = pm[__float_as_int(e1.y) & 0xfff];
      if (v0) lt[j16] = make_float2(e0.x, __int_as_float(i0));
      if (v1) lt[j16 + 16] = make_float2(e1.x, __int_as_float(i1));
      const int maxc = max(max(__builtin_amdgcn_readlane(cn, 0), __builtin_amdgcn_readlane(cn, 16)),
                           max(__builtin_amdgcn_readlane(cn, 32), __builtin_amdgcn_readlane(cn, 48)));
      int r0 = 0, r1 = 0;
      float vmax = kLowest;
      for (int i = 0; i < maxc; ++i) {
        const float2 e = lt[i];
        const bool okc = i < cn;
        const int ie = __float_as_int(e.y);
        r0 += (okc && beats(e.x, ie, e0.x, i0)) ? 1 : 0;
        r1 += (okc && beats(e.x, ie, e1.x, i1)) ? 1 : 0;
        vmax = okc ? fmaxf(vmax, e.x) : vmax;
      }
      const bool s0 = v0 && r0 < k, s1 = v1 && r1 < k;
      float g0, g1, lse = 0.f;
      if constexpr (FULL) {
        const float2 mz = *(const float2*)(lds + L::kMZ + ((par * 32 + nloc) * 16 + j16) * 8);
        const float mm = row16_max(mz.x);
        const float zz = row16_sum(mz.y * __builtin_amdgcn_exp2f((mz.x - mm) * kLog2e));
        lse = mm + __builtin_amdgcn_logf(zz) * kLn2;
        g0 = __builtin_amdgcn_exp2f((e0.x - lse) * kLog2e);
        g1 = __builtin_amdgcn_exp2f((e1.x - lse) * kLog2e);
      } else {
        // Fig. 12: softmax over the k selected logits, max subtracted; the
        // denominator is summed in rank order (slots 0..k-1 of the token's log,
        // free once every lane holds its entries), so it does not depend on the
        // order in which the candidates were logged
        const float w0 = s0 ? __builtin_amdgcn_exp2f((e0.x - vmax) * kLog2e) : 0.f;
        const float w1 = s1 ? __builtin_amdgcn_exp2f((e1.x - vmax) * kLog2e) : 0.f;
        float* wr = (float*)lt;
        if (s0) wr[r0] = w0;
        if (s1) wr[r1] = w1;
        const float4 wa = *(const float4*)wr, wb = *(const float4*)(wr + 4);
        const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
        float den = 0.f;
#pragma unroll
        for (int j = 0; j < kSlK; ++j) den += (j < k) ? wv[j] : 0.f;
        const float inv = 1.f / den;
        g0 = w0 * inv;
        g1 = w1 * inv;
      }
      if (n < a.N) {
        const size_t o = (size_t)n * k;
        if (s0) {
          stage[nloc * kSlK + r0] = make_int2(i0, __float_as_int(g0));
          if (a.out_logit) a.out_logit[o + r0] = e0.x;
        }
        if (s1) {
          stage[nloc * kSlK + r1] = make_int2(i1, __float_as_int(g1));
          if (a.out_logit) a.out_logit[o + r1] = e1.x;
        }
        if (FULL && j16 == 0 && !ovf && a.out_lse) a.out_lse[n] = lse;
      }
      // overflowed tokens of this wave: slow exact path (lane column = token)
      const uint64_t om = __builtin_amdgcn_ballot_w64(ovf && j16 == 0);
      if (om != 0) {
        uint32_t tok_mask = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if ((om >> (16 * t)) & 1) tok_mask |= 1u << (4 * c + t);
        const long long n0 = ((long long)blockIdx.x + (long long)jj * sa.G) * kTile;
        sl_slow<FULL, BIAS, R16>(a, zs, stage, lane, tok_mask, n0);
      }
    }
  }
  if (nbw > 0) copy_out(nbw - 1);
}

template <bool FULL, bool BIAS, int R16, int TV, int NZ, int D, bool TAIL>
__global__ __launch_bounds__(64 * kSlWaves) void slice_kernel(SlArgs sa) {
  typedef SlLds<FULL, BIAS, R16, TV, NZ> L;
  extern __shared__ __align__(16) char sl_lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // stage the bias (accumulator layout) and the 16-bit expert of every sweep
  // position; clear the flags and counters
  if constexpr (BIAS) {
    const float4* src = (const float4*)sa.base.biasp;
    float4* dst = (float4*)(sl_lds + L::kBias);
    for (int i = threadIdx.x; i < kSlNT * 8; i += 64 * kSlWaves) dst[i] = src[i];
  }
  {
    const int2* src = (const int2*)sa.base.perm;
    uint32_t* dst = (uint32_t*)(sl_lds + L::kPerm);
    for (int i = threadIdx.x; i < kSlNT * 16; i += 64 * kSlWaves) {
      const int2 p = src[i];
      dst[i] = (uint32_t)(p.x & 0xffff) | ((uint32_t)p.y << 16);
    }
  }
  if (threadIdx.x < 256) ((int*)sl_lds)[threadIdx.x] = 0;   // flags, stats, counters
  __syncthreads();
  const int nbw = (sa.NB - (int)blockIdx.x + sa.G - 1) / sa.G;   // blocks of this workgroup
  if (wave < kPcProd)
    produce_z<R16, D, TAIL>(ProdArgs{sa.base.X, sa.base.N, sa.base.h, sa.R1q, sa.KSP, sa.G},
                            SlHandOff<R16, NZ>{sl_lds, sa.spin_limit}, wave, lane, nbw);
  else
    sl_consume<FULL, BIAS, R16, TV, NZ>(sa, sl_lds, wave - kPcProd, lane, nbw);
}

}  // namespace more
