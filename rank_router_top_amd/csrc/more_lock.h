// more_lock.h -- workgroup-lockstep streaming form of the fused low-rank router
// (bf16 storage, k <= 8, r <= 64, M <= 65536) for gfx950.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.1 Algorithm 1 (phase 1: z = X-block times the
// down-projection on chip; phase 2: one sweep over the experts with a running
// top-k; only N x k results are written).  Two consecutive token blocks are
// overlapped per wave -- phase 2 of block i runs while phase 1 of block i+1
// streams X -- as in more_stream.h, with three MI355X-specific changes:
//
//  * X is read with fully coalesced 16-byte loads (whole 128-byte lines per
//    row) and transposed into the MFMA operand layout through a small per-wave
//    LDS buffer.  Reading it directly in operand layout (two 16-byte pieces
//    of 32 different rows per instruction) streams about 15% slower on
//    MI355X HBM3E.
//  * The weight operands of each batch (R1 K-steps, R2 tiles, bias) are staged
//    once per workgroup into a double-buffered LDS area shared by its 8 waves,
//    which therefore walk the same batch schedule in lockstep (one barrier per
//    batch).  The sweep reads operands only from LDS.
//  * Every global load of batch j+1 (the wave's X chunk and its share of the
//    weight staging) is issued during batch j and consumed at the start of
//    batch j+1.  Vector-memory loads complete in order, so keeping the
//    short-latency operand reads out of that counter is what lets the HBM
//    stream stay in flight across a whole batch.
//
// Batch schedule per block iteration: NBATCH batches; batch j covers K-steps
// [K(j), K(j+1)) of the next block's phase 1 and tiles [T(j), T(j+1)) of the
// current block's sweep, with K(j) = j*KS/NBATCH and T(j) = j*NT/NBATCH
// (at most KPBM K-steps and TPBM tiles per batch).
#pragma once
#include "more_device.h"
#include "more_lowrank.h"
#include "more_pack.h"

namespace more {

struct LockArgs {
  LowRankArgs base;   // X, N, h, NT, k, packed weights, outputs
  int NB;             // token blocks of 32
  int G;              // waves in the grid (8 per workgroup)
  int NI;             // block iterations: ceil(NB / G)
  int NBATCH;         // batches per block
  int KS;             // K-steps of the down-projection
};

// Compact log for the lockstep kernel: values and 16-bit sweep positions in
// two arrays, 6 bytes per entry (positions < 65536).
struct Log6 {
  float* val;      // [CAP][64]
  uint16_t* pos;   // [CAP][64]
};

template <int KMAX, int CAP>
struct LockState {
  float L[KMAX];
  float thr_p, thr;
  int cnt;
  float m, Z;
  __device__ __forceinline__ void init(int k) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) L[j] = (j < KMAX - k) ? __builtin_inff() : kLowest;
    thr_p = kLowest;
    thr = kLowest;
    cnt = 0;
    m = kLowest * 0.25f;
    Z = 0.f;
  }
};

// Out of line (rare): drop log entries below thr; when exact ties at thr keep
// the log nearly full, keep only the k ties of lowest expert index.
__device__ __noinline__ int compact_log6(float* val, uint16_t* pos, int lane, int cnt, float thr,
                                         const int* __restrict__ perm, int k, int cap) {
  int w = 0;
  for (int c = 0; c < cnt; ++c) {
    const float v = val[c * kWave + lane];
    const uint16_t p = pos[c * kWave + lane];
    if (v >= thr) {
      val[w * kWave + lane] = v;
      pos[w * kWave + lane] = p;
      ++w;
    }
  }
  cnt = w;
  if (any_lane(cnt > cap - 8)) {
    if (cnt > cap - 8) {
      for (int c = 0; c < cnt; ++c) {
        const float v = val[c * kWave + lane];
        if (v == thr) {
          const int oi = perm[pos[c * kWave + lane]];
          int rank = 0;
          for (int c2 = 0; c2 < cnt; ++c2)
            if (val[c2 * kWave + lane] == thr && perm[pos[c2 * kWave + lane]] < oi) ++rank;
          if (rank >= k) val[c * kWave + lane] = -__builtin_inff();
        }
      }
      w = 0;
      for (int c = 0; c < cnt; ++c) {
        const float v = val[c * kWave + lane];
        const uint16_t p = pos[c * kWave + lane];
        if (v >= thr) {
          val[w * kWave + lane] = v;
          pos[w * kWave + lane] = p;
          ++w;
        }
      }
      cnt = w;
    }
  }
  return cnt;
}

template <int KMAX, int CAP, bool FULL>
__device__ __forceinline__ void lock_tile(LockState<KMAX, CAP>& st, const floatx16& acc, int pos_base,
                                          Log6 lg, int lane, bool hi_half, const int* __restrict__ perm,
                                          int k) {
  float g[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    g[q] = fmaxf(fmaxf(acc[4 * q], acc[4 * q + 1]), fmaxf(acc[4 * q + 2], acc[4 * q + 3]));
  const float tmax = fmaxf(fmaxf(g[0], g[1]), fmaxf(g[2], g[3]));
  if (FULL) {
    const float mn = fmaxf(st.m, tmax);
    const float mb = mn * kLog2e;
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) s += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], kLog2e, -mb));
    st.Z = st.Z * __builtin_amdgcn_exp2f((st.m - mn) * kLog2e) + s;
    st.m = mn;
  }
  st.thr_p = partner_f32(st.L[KMAX - 1], hi_half);
  st.thr = fmaxf(st.L[KMAX - 1], st.thr_p);
  if (any_lane(tmax >= st.thr)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (any_lane(g[q] >= st.thr)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = acc[4 * q + e];
          if (x >= st.thr) {
#pragma unroll
            for (int j = KMAX - 1; j >= 1; --j) st.L[j] = __builtin_amdgcn_fmed3f(st.L[j - 1], st.L[j], x);
            st.L[0] = fmaxf(st.L[0], x);
            lg.val[st.cnt * kWave + lane] = x;
            lg.pos[st.cnt * kWave + lane] = (uint16_t)(pos_base + 8 * q + e);
            ++st.cnt;
            st.thr = fmaxf(st.L[KMAX - 1], st.thr_p);
          }
        }
        if (any_lane(st.cnt > CAP - 4)) st.cnt = compact_log6(lg.val, lg.pos, lane, st.cnt, st.thr, perm, k, CAP);
      }
    }
  }
}

template <int KMAX, int CAP, bool FULL>
__device__ __forceinline__ void lock_finish(LockState<KMAX, CAP>& st, Log6 lg, int lane, bool hi_half,
                                            bool rowok, long long n, const int* __restrict__ perm, int k,
                                            int* out_idx, float* out_gate, float* out_logit,
                                            float* out_lse) {
  st.thr_p = partner_f32(st.L[KMAX - 1], hi_half);
  st.thr = fmaxf(st.L[KMAX - 1], st.thr_p);
  st.cnt = compact_log6(lg.val, lg.pos, lane, st.cnt, st.thr, perm, k, CAP);
  const int cnt_p = (int)partner_u32((uint32_t)st.cnt, hi_half);
  float lse = 0.f;
  if (FULL) {
    const float mp = partner_f32(st.m, hi_half), Zp = partner_f32(st.Z, hi_half);
    const float mm = fmaxf(st.m, mp);
    const float Zt = st.Z * __builtin_amdgcn_exp2f((st.m - mm) * kLog2e) +
                     Zp * __builtin_amdgcn_exp2f((mp - mm) * kLog2e);
    lse = mm + __builtin_amdgcn_logf(Zt) * kLn2;
  }
  if (hi_half || !rowok) return;
  float V[KMAX];
  int IX[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    V[j] = -__builtin_inff();
    IX[j] = 0x7fffffff;
  }
  for (int c = 0; c < st.cnt; ++c)
    ordered_insert<KMAX>(V, IX, lg.val[c * kWave + lane], perm[lg.pos[c * kWave + lane]]);
  for (int c = 0; c < cnt_p; ++c)
    ordered_insert<KMAX>(V, IX, lg.val[c * kWave + lane + 32], perm[lg.pos[c * kWave + lane + 32]]);
  float w[KMAX];
  if (FULL) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) w[j] = __builtin_amdgcn_exp2f((V[j] - lse) * kLog2e);
  } else {
    float denom = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      w[j] = (j < k) ? __builtin_amdgcn_exp2f((V[j] - V[0]) * kLog2e) : 0.f;
      denom += w[j];
    }
    const float inv = 1.f / denom;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) w[j] *= inv;
  }
  const size_t o = (size_t)n * k;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      out_idx[o + j] = IX[j];
      out_gate[o + j] = w[j];
      if (out_logit) out_logit[o + j] = V[j];
    }
  }
  if (FULL && out_lse) out_lse[n] = lse;
}

constexpr int kLockWaves = 8;

// LDS footprint of the lockstep kernel (bytes).
template <int KMAX, int R16, int KPBM, int TPBM>
struct LockLds {
  static constexpr int CAP = 2 * KMAX + 8;
  static constexpr int RB = (R16 + 1) / 2;
  static constexpr int XRS = 32 * KPBM + 16;                        // X row stride (padded)
  static constexpr int XBUF = 32 * XRS;                             // per wave
  static constexpr int NCH = KPBM * RB + TPBM * R16 + (TPBM + 3) / 4;  // 1 KiB chunks per batch
  static constexpr int SBUF = NCH * 1024;                           // shared, per slot
  static constexpr int LOGV = CAP * kWave * 4, LOGP = CAP * kWave * 2;
  static constexpr int total = kLockWaves * (XBUF + LOGV + LOGP) + 2 * SBUF;
};

template <int KMAX, bool FULL, int R16, int KPBM, int TPBM>
__global__ __launch_bounds__(64 * kLockWaves) __attribute__((amdgpu_waves_per_eu(2)))
void lock_kernel(LockArgs la) {
  static_assert(TPBM <= 4 && (TPBM % 2) == 0, "bias staging covers 4 tiles; tiles run in pairs");
  static_assert(32 % KPBM == 0, "X chunk rows per instruction");
  using LD = LockLds<KMAX, R16, KPBM, TPBM>;
  constexpr int CAP = LD::CAP, RB = LD::RB, NCH = LD::NCH;
  constexpr int SPW = (NCH + kLockWaves - 1) / kLockWaves;          // staged chunks per wave
  const LowRankArgs& a = la.base;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool hi = lane >= 32;
  const int hf = hi ? 1 : 0, col = lane & 31;
  const int gw = blockIdx.x * kLockWaves + wave;
  uint8_t* xbuf = smem + wave * LD::XBUF;
  uint8_t* sbuf = smem + kLockWaves * LD::XBUF;                     // 2 slots
  Log6 lg{(float*)(sbuf + 2 * LD::SBUF + wave * (LD::LOGV + LD::LOGP)),
          (uint16_t*)(sbuf + 2 * LD::SBUF + wave * (LD::LOGV + LD::LOGP) + LD::LOGV)};
  const uint8_t* X = (const uint8_t*)a.X;
  const size_t rowb = (size_t)a.h * 2;
  const int NB = la.NB, NBATCH = la.NBATCH, KS = la.KS, NT = a.NT;

  // ------------------------------------------------------------ staging loads
  // X chunk of batch (i, j): block b = gw + i*G, K-steps K(j)..K(j)+KPBM-1,
  // coalesced: instruction q covers rows q*(32/KPBM) .. +32/KPBM-1, each row a
  // contiguous 32*KPBM-byte piece split over 2*KPBM lanes.
  constexpr int LPR = 2 * KPBM, RPI = 32 / KPBM;                    // lanes per row, rows per instr
  const int xr_row = lane / LPR, xr_col = 16 * (lane % LPR);
  bf16x8 xs[KPBM];
  u32x4 ws[SPW];
  auto issue = [&](int i, int j) {
    const int b = gw + i * la.G;
    const bool blk = (i < la.NI) && (b < NB);
    const int k0 = j * KS / NBATCH;
#pragma unroll
    for (int q = 0; q < KPBM; ++q) {
      long long row = (long long)b * kTile + q * RPI + xr_row;
      row = row < a.N ? row : a.N - 1;
      int cb = 32 * k0 + xr_col;                                    // byte column in the row
      cb = (cb + 16 <= (int)rowb) ? cb : 0;                         // past the row end: any valid piece
      const bf16x8* p = blk ? (const bf16x8*)(X + (size_t)row * rowb + cb) : (const bf16x8*)X;
      xs[q] = __builtin_nontemporal_load(p);
    }
    // shared weight chunks of batch j: R1 K-steps, R2 tiles, bias
    const int t0 = j * NT / NBATCH;
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int c = wave + u * kLockWaves;
      const u32x4* src = (const u32x4*)a.R1p;                       // any valid address by default
      if (c < KPBM * RB) {
        int s = k0 + c / RB;
        s = s < KS ? s : KS - 1;
        src = (const u32x4*)a.R1p + ((size_t)s * RB + c % RB) * kWave;
      } else if (c < KPBM * RB + TPBM * R16) {
        const int cc = c - KPBM * RB;
        int t = t0 + cc / R16;
        t = t < NT ? t : NT - 1;
        src = (const u32x4*)a.R2p + ((size_t)t * R16 + cc % R16) * kWave;
      } else if (c < NCH) {
        const int cc = c - KPBM * RB - TPBM * R16;
        int t = t0 + 4 * cc;
        t = t + 4 <= NT ? t : (NT >= 4 ? NT - 4 : 0);               // bias of 4 tiles = 1 KiB
        src = (const u32x4*)(a.biasq + (size_t)t * kWave);           // 4 tiles x 256 B
      }
      ws[u] = src[lane];
    }
  };
  // Bias tiles staged per batch start at tile bias_t0(j) (aligned as above).
  auto bias_t0 = [&](int j) {
    const int t0 = j * NT / NBATCH;
    return t0 + 4 <= NT ? t0 : (NT >= 4 ? NT - 4 : 0);
  };
  auto commit = [&](int j) {                                        // VGPR staging -> LDS
#pragma unroll
    for (int q = 0; q < KPBM; ++q)
      *(bf16x8*)(xbuf + (q * RPI + xr_row) * LD::XRS + xr_col) = xs[q];
    uint8_t* slot = sbuf + (j & 1) * LD::SBUF;
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int c = wave + u * kLockWaves;
      if (c < NCH) *(u32x4*)(slot + c * 1024 + 16 * lane) = ws[u];
    }
  };

  // --------------------------------------------------------------- compute
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)((!hi && e < 2) ? 1.f : 0.f);
  bf16x8 zh[R16], zl[R16];
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
  auto logits = [&](const uint8_t* slot, int tl, int bias_tl) {   // tile tl of this batch
    const uint8_t* r2 = slot + (KPBM * RB + tl * R16) * 1024 + 16 * lane;
    const uint32_t bw = *(const uint32_t*)(slot + (KPBM * RB + TPBM * R16) * 1024 + bias_tl * 256 + 4 * lane);
    bf16x8 ab;
#pragma unroll
    for (int e = 0; e < 8; ++e) ab[e] = (bf16)0.f;
    ab[0] = __builtin_bit_cast(bf16, (uint16_t)(bw & 0xffffu));
    ab[1] = __builtin_bit_cast(bf16, (uint16_t)(bw >> 16));
    floatx16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    acc = mfma_bf16(ab, ones, acc);
    bf16x8 w[R16];
#pragma unroll
    for (int m = 0; m < R16; ++m) w[m] = *(const bf16x8*)(r2 + m * 1024);
#pragma unroll
    for (int m = 0; m < R16; ++m) acc = mfma_bf16(w[m], zh[m], acc);
#pragma unroll
    for (int m = 0; m < R16; ++m) acc = mfma_bf16(w[m], zl[m], acc);
    return acc;
  };

  LockState<KMAX, CAP> st;
  issue(0, 0);                                                      // block 0, batch 0
  for (int i = -1; i < la.NI; ++i) {
    const int bcur = gw + i * la.G;
    const bool has_cur = i >= 0 && bcur < NB;                       // wave-uniform
    const bool has_nxt = (i + 1 < la.NI) && (gw + (i + 1) * la.G < NB);
    if (has_cur) st.init(a.k);
    for (int j = 0; j < NBATCH; ++j) {
      commit(j);
      __syncthreads();
      const uint8_t* slot = sbuf + (j & 1) * LD::SBUF;
      // phase 1 of block i+1: K-steps K(j) .. K(j+1)-1
      const int k0 = j * KS / NBATCH, k1 = (j + 1) * KS / NBATCH;
      if (has_nxt) {
#pragma unroll
        for (int u = 0; u < KPBM; ++u) {
          if (k0 + u < k1) {
            const bf16x8 xv = *(const bf16x8*)(xbuf + col * LD::XRS + 32 * u + 16 * hf);
#pragma unroll
            for (int b = 0; b < RB; ++b) {
              const bf16x8 rv = *(const bf16x8*)(slot + (u * RB + b) * 1024 + 16 * lane);
              zacc[b] = mfma_bf16(rv, xv, zacc[b]);
            }
          }
        }
      }
      // loads for the next batch (or batch 0 of the next block iteration)
      if (j + 1 < NBATCH) issue(i + 1, j + 1);
      else issue(i + 2, 0);
      // phase 2 of block i: tiles T(j) .. T(j+1)-1 (at most TPBM), two in flight
      if (has_cur) {
        const int t0 = j * NT / NBATCH, nt = (j + 1) * NT / NBATCH - t0;
        const int bt = t0 - bias_t0(j);
        floatx16 accA = logits(slot, 0, bt), accB;
#pragma unroll
        for (int tl = 0; tl < TPBM; tl += 2) {
          if (tl + 1 < nt) accB = logits(slot, tl + 1, bt + tl + 1);
          if (tl < nt) lock_tile<KMAX, CAP, FULL>(st, accA, kTile * (t0 + tl) + 4 * hf, lg, lane, hi, a.perm, a.k);
          if (tl + 2 < nt) accA = logits(slot, tl + 2, bt + tl + 2);
          if (tl + 1 < nt) lock_tile<KMAX, CAP, FULL>(st, accB, kTile * (t0 + tl + 1) + 4 * hf, lg, lane, hi, a.perm, a.k);
        }
      }
    }
    if (has_cur) {
      const long long n = (long long)bcur * kTile + col;
      lock_finish<KMAX, CAP, FULL>(st, lg, lane, hi, n < a.N, n, a.perm, a.k, a.out_idx, a.out_gate,
                                   a.out_logit, a.out_lse);
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
