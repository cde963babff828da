// more_sweep.h -- expert sweep of the low-rank router with the up-projection
// tiles shared through an LDS ring (gfx950).
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.1 Algorithm 1 (per token block, one sweep over the expert
// tiles of z R2 with a running top-k; only the N x k results reach memory),
// Fig. 12 and App. F.2.1 eq. (6)/(8) for the gates and the running normaliser.
//
// Input: z of every 32-token block as bf16 hi + lo parts in the B-operand
// layout of v_mfma_f32_32x32x16_bf16 (written by the projection kernel).
//
// Why a shared ring.  Each 32-expert tile of R2 (R16 KiB) is an MFMA operand
// for every token block.  Read from L2 by each wave separately it would cost
// 1 KiB of L2 traffic per 32x32x16 MFMA, i.e. ~250 GB/s per CU at the MFMA
// rate, far above what a CU draws from L2 (~70-100 GB/s measured).  Here one
// loader wave per workgroup copies every tile once into an LDS ring
// (buffer_load ... lds, no registers involved) and the NC consumer waves, each
// routing its own 32-token block, read the operands from LDS (~250 B/clk per
// CU available).  All consumers sweep the same tile sequence, so a slot is
// refilled once every consumer has read it: the ring (RING tiles) absorbs the
// consumers' different speeds.
//
// Exact top-k per token (ties to the lower expert index):
//   seed pass (the first P tiles of the sweep order -- bias descending, so they
//     hold most winners -- or every tile without a bias): hi-only logits
//     z_hi R2 (R16 MFMAs per tile, no bias); per lane and tile the maximum plus
//     the smallest bias of the tile is at most the logit of one real expert
//     (up to eps below); each lane keeps the k largest of these (v_med3 list),
//     and the two lanes of a token merge theirs: thr = k-th largest - eps is a
//     lower bound of the token's k-th exact logit.  eps bounds |exact - hi-only|
//     per token: ||z_lo|| max_m ||R2[:, m]|| (the dropped z_lo term,
//     Cauchy-Schwarz) + 2^-15 (||z_hi|| max_m ||R2[:, m]|| + max |b|), which
//     covers the fp32 accumulation of either MFMA chain and the bf16 hi + lo
//     representation of the bias.
//   main sweep (every tile): exact logits, bias included, from 2 R16 + 1 MFMAs
//     (z_hi, z_lo, and the bias as a bf16 hi + lo operand against a ones
//     operand); a 4-logit group whose maximum reaches thr is appended to the
//     lane's log (16 bytes + a 16-bit sweep position).  Every top-k logit is
//     >= thr, so it is logged.  When a lane's log is nearly full -- and once
//     after the first kTightenTile main tiles, where the high-bias winners
//     are -- the whole wave tightens: thr rises to the token's k-th largest
//     logged group maximum (each is the exact logit of a distinct expert, so
//     still a lower bound of the k-th logit) and groups below it are dropped.
//   finish: the token's k largest logged logits (v_med3 lists merged across
//     the two lanes) give the k-th value; each lane writes the sweep position
//     of each of its selected logits at its rank; exact ties fall back to an
//     ordered merge by (logit desc, expert index asc).  Positions become expert
//     indices through the sweep order, gates follow Fig. 12 or eq. (6).
#pragma once
#include "more_device.h"
#include "more_pc.h"
#include "more_twopass.h"

namespace more {

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const uint32_t lds_cu32;

constexpr int kTightenTile = 32;   // main-sweep tiles before the scheduled tightening

struct SweepArgs {
  const void* Z;             // [NB][hi, lo][R16][64 lanes][16 B]: z of every 32-token block
  const void* R2p;           // [NT][R16][64 lanes][16 B]: A operands, sweep order
  const uint32_t* biasq;     // [NT][64]: (b_hi | b_lo << 16) of row l in lane l < 32, 0 above
  const float* bmin;         // [NT]: smallest bias of the tile's experts (-inf if it has padding)
  const float* wstat;        // [3]: max_m ||R2[:, m]||_2, max_m |b_m|, seed tiles P (int bits, 1 <= P <= NT)
  const int* perm;           // [Mpad]: sweep position -> expert
  long long N;
  int NB, NT, k;              // blocks, tiles, k
  int* out_idx;
  float* out_gate;
  float* out_logit;          // may be null
  float* out_lse;            // may be null (written in LSE mode)
  int* status;               // device word set to a nonzero code if a bounded wait gave up
  int spin_limit;            // polls before a wait gives up
};

// LDS map.  Flag words (ints): published (tiles of the sequence in the ring
// so far; tile g sits in slot g % RING), prog[NC] (tiles each consumer has
// finished reading), abort.
template <int R16, int NC, int RING, int CAP, int KMAX>
struct SwLds {
  static constexpr int TB = R16 * 1024 + 256;   // ring slot: R16 A operands + 64 bias words
  static constexpr int kPub = 0, kProg = 1, kAbort = 1 + NC;
  static_assert(NC + 2 <= 64, "flag words");
  static constexpr int kRing = 256;
  static constexpr int kCons = kRing + RING * TB;
  static constexpr int kLogV = 0;                        // [CAP][64] 4 logits (16 B)
  static constexpr int kLogP = CAP * 1024;               // [CAP][64] u16 sweep positions
  static constexpr int kStage = kLogP + CAP * 128;       // TpStage<KMAX> words
  // the result block, plus 1 KiB so that every 16-byte read of its arrays stays inside
  static constexpr int kConsBytes = (kStage + TpStage<KMAX>::kWords * 4 + 1024 + 15) / 16 * 16;
  static constexpr int bytes = kCons + NC * kConsBytes;
};

struct SwLog {
  lds_f4* val;    // entry c of lane l: val[c * 64 + l]
  lds_u16* pos;   // pos[c * 64 + l]: sweep position of the group's first logit
};

// s_waitcnt with vmcnt = n (n < 64), expcnt and lgkmcnt at their maxima (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Record a given-up bounded wait for the host (status word in the caller's
// workspace; the routing call's check entry point reads it).
__device__ __forceinline__ void sw_fail(int* status, int code) {
  if (status) __hip_atomic_store(status, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tightening (whole wave active, called uniformly).  thr rises to the token's
// k-th largest logged group maximum; groups whose maximum is below the new thr
// are dropped.  If exact ties at thr still leave a lane's log nearly full, the
// tied logits of that lane are cut to the k of lowest expert index (the others
// can never be selected).
// Takes and returns (thr, count) by value: a reference to the caller's state
// would force that state into scratch memory around the hot loop.
template <int KMAX, int CAP>
__device__ __noinline__ float2 sw_tighten(float thr, int cnt, SwLog lg, int lane, bool hi_half, int k,
                                          const int* __restrict__ perm) {
  float L[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) L[j] = (j < KMAX - k) ? __builtin_inff() : kLowest;
  for (int c = 0; c < cnt; ++c) {
    const floatx4 v = lg.val[c * kWave + lane];
    med3_insert<KMAX>(L, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  }
  float T[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) T[j] = L[j];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const float p = partner_f32(L[j], hi_half);
    med3_insert<KMAX>(T, j >= KMAX - k ? p : kLowest);
  }
  const float t2 = fmaxf(thr, T[KMAX - 1]);
  int w = 0;
  for (int c = 0; c < cnt; ++c) {
    const floatx4 v = lg.val[c * kWave + lane];
    if (fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])) >= t2) {
      const uint16_t p = lg.pos[c * kWave + lane];
      lg.val[w * kWave + lane] = v;
      lg.pos[w * kWave + lane] = p;
      ++w;
    }
  }
  if (w > CAP - 2) {
    // exact ties at t2 keep the log full: keep the (k - #above) tied logits of
    // lowest expert index, then squeeze
    int gt = 0;
    for (int c = 0; c < w; ++c) {
      const floatx4 v = lg.val[c * kWave + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) gt += v[e] > t2 ? 1 : 0;
    }
    const int keep = k - gt;
    for (int c = 0; c < w; ++c) {
      floatx4 v = lg.val[c * kWave + lane];
      const int p = lg.pos[c * kWave + lane];
      bool changed = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (v[e] == t2) {
          const int oi = perm[p + e];
          int rank = 0;
          for (int c2 = 0; c2 < w; ++c2) {
            const floatx4 v2 = lg.val[c2 * kWave + lane];
            const int p2 = lg.pos[c2 * kWave + lane];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2)
              if (v2[e2] == t2 && perm[p2 + e2] < oi) ++rank;
          }
          if (rank >= keep) {
            v[e] = -__builtin_inff();
            changed = true;
          }
        }
      }
      if (changed) lg.val[c * kWave + lane] = v;
    }
    int w2 = 0;
    for (int c = 0; c < w; ++c) {
      const floatx4 v = lg.val[c * kWave + lane];
      if (fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])) >= t2) {
        const uint16_t p = lg.pos[c * kWave + lane];
        lg.val[w2 * kWave + lane] = v;
        lg.pos[w2 * kWave + lane] = p;
        ++w2;
      }
    }
    w = w2;
  }
  return make_float2(t2, __int_as_float(w));
}

// Main-sweep logging of one tile (acc: this lane's 16 exact logits, bias
// included, -inf on padding rows; pos_base = 32 t + 4 hf; register 4q + e is
// sweep row 8q + 4hf + e).  Appends are branch-free inside a group that has a
// candidate in some lane: every lane writes slot cnt, only a hit advances it.
template <int KMAX, int CAP>
__device__ __forceinline__ void sw_log_tile(TwoPassState<KMAX>& st, const floatx16& acc, int pos_base, SwLog lg,
                                            int lane, bool hi_half, int k, const int* __restrict__ perm) {
  floatx4 g;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    g[q] = fmaxf(fmaxf(acc[4 * q], acc[4 * q + 1]), fmaxf(acc[4 * q + 2], acc[4 * q + 3]));
  const float tmax = fmaxf(fmaxf(g[0], g[1]), fmaxf(g[2], g[3]));
  if (any_lane(tmax >= st.thr)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (any_lane(g[q] >= st.thr)) {
        if (any_lane(st.cnt >= CAP)) {
          const float2 r = sw_tighten<KMAX, CAP>(st.thr, st.cnt, lg, lane, hi_half, k, perm);
          st.thr = r.x;
          st.cnt = __float_as_int(r.y);
        }
        lg.val[st.cnt * kWave + lane] = floatx4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        lg.pos[st.cnt * kWave + lane] = (uint16_t)(pos_base + 8 * q);
        st.cnt += (g[q] >= st.thr) ? 1 : 0;
      }
    }
    // the appends complete here, so later LDS waits need not count them
    lds_drain();
  }
}

// Exact ordering of the logged candidates (rare: exact ties decide ranks):
// ordered insertion by (logit desc, expert asc) over both lanes' logs; the
// sweep positions and logits of the k first go to the token's rows of the
// result block (idx and logit words).  Results go through LDS, not through
// pointers to the caller's registers, which would move those into scratch.
template <int KMAX>
__device__ __noinline__ void sw_order_slow(SwLog lg, int lane, int cnt, int cnt_p, float thr,
                                           const int* __restrict__ perm, int k, lds_f32* stg) {
  typedef TpStage<KMAX> S;
  float v8[KMAX];
  int i8[KMAX], p8[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    v8[j] = -__builtin_inff();
    i8[j] = 0x7fffffff;
    p8[j] = 0;
  }
  for (int h = 0; h < 2; ++h) {
    const int ln = lane + 32 * h, n = h ? cnt_p : cnt;
    for (int c = 0; c < n; ++c) {
      const floatx4 v = lg.val[c * kWave + ln];
      const int p = lg.pos[c * kWave + ln];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (v[e] >= thr) {
          const float x = v[e];
          const int ix = perm[p + e];
          bool cc[KMAX];
#pragma unroll
          for (int j = 0; j < KMAX; ++j) cc[j] = (x > v8[j]) || (x == v8[j] && ix < i8[j]);
#pragma unroll
          for (int j = KMAX - 1; j >= 1; --j) {
            const bool tj = cc[j - 1], sj = cc[j];
            const float nv = tj ? v8[j - 1] : (sj ? x : v8[j]);
            const int ni = tj ? i8[j - 1] : (sj ? ix : i8[j]);
            const int np = tj ? p8[j - 1] : (sj ? p + e : p8[j]);
            v8[j] = nv;
            i8[j] = ni;
            p8[j] = np;
          }
          if (cc[0]) {
            v8[0] = x;
            i8[0] = ix;
            p8[0] = p + e;
          }
        }
      }
    }
  }
  const int o = (lane & 31) * k;
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k) {
      stg[S::kIdx + o + j] = __int_as_float(p8[j]);
      stg[S::kLogit + o + j] = v8[j];
    }
}

// End of a token block: results of the 32 tokens into the wave's result block
// `stg` (TpStage layout); the idx words hold SWEEP POSITIONS here (converted
// to expert indices by the caller).  Whole wave active on entry.
template <int KMAX, bool FULL, bool LSE>
__device__ __forceinline__ void sw_finish(const TwoPassState<KMAX>& st, SwLog lg, int lane, bool hi_half,
                                          const int* __restrict__ perm, int k, bool want_logit, lds_f32* stg) {
  static_assert(LSE || !FULL, "the full-softmax gate needs the normaliser");
  typedef TpStage<KMAX> S;
  const int cnt_p = (int)partner_u32((uint32_t)st.cnt, hi_half);
  const float thr = fmaxf(st.thr, partner_f32(st.thr, hi_half));
  float lse = 0.f;
  if (LSE) {
    // eq. (8) across the two halves of the token
    const float mp = partner_f32(st.m, hi_half), Zp = partner_f32(st.Z, hi_half);
    const float mm = fmaxf(st.m, mp);
    const float Zt = st.Z * __builtin_amdgcn_exp2f((st.m - mm) * kLog2e) +
                     Zp * __builtin_amdgcn_exp2f((mp - mm) * kLog2e);
    lse = mm + __builtin_amdgcn_logf(Zt) * kLn2;
  }
  // 1. the token's k largest logged logits: each lane's own (v_med3 list),
  //    merged across the two lanes
  float L[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) L[j] = (j < KMAX - k) ? __builtin_inff() : kLowest;
#pragma unroll 2
  for (int c = 0; c < st.cnt; ++c) {
    const floatx4 v = lg.val[c * kWave + lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) med3_insert<KMAX>(L, v[e]);
  }
  float T[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) T[j] = L[j];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const float p = partner_f32(L[j], hi_half);
    med3_insert<KMAX>(T, j >= KMAX - k ? p : kLowest);
  }
  const float vk = T[KMAX - 1];
  // 2. without exact ties a selected logit's rank is the number of selected
  //    logits above it: each lane writes the sweep position of its own
  //    selected logits at their rank
  const int tok = lane & 31;
  const int o = tok * k;
  int nge = 0;
#pragma unroll 2
  for (int c = 0; c < st.cnt; ++c) {
    const floatx4 v = lg.val[c * kWave + lane];
    const int p = lg.pos[c * kWave + lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (v[e] >= vk) {
        ++nge;
        int r = -(KMAX - k);   // the +inf pads count as larger
#pragma unroll
        for (int j = 0; j < KMAX; ++j) r += T[j] > v[e] ? 1 : 0;
        if (r < k) stg[S::kIdx + o + r] = __int_as_float(p + e);
      }
    }
  }
  bool tie = nge + (int)partner_u32((uint32_t)nge, hi_half) != k;
#pragma unroll
  for (int j = 0; j + 1 < KMAX; ++j) tie = tie || (j >= KMAX - k && T[j] == T[j + 1]);
  float V[KMAX];
  if (!any_lane(tie)) {
    if (hi_half) return;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) V[j] = T[(j + KMAX - k) < KMAX ? (j + KMAX - k) : KMAX - 1];
  } else {
    if (hi_half) return;
    sw_order_slow<KMAX>(lg, lane, st.cnt, cnt_p, thr, perm, k, stg);
    lds_drain();
#pragma unroll
    for (int j = 0; j < KMAX; ++j) V[j] = (j < k) ? stg[S::kLogit + o + j] : -__builtin_inff();
  }
  float wgt[KMAX];
  if (FULL) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) wgt[j] = __builtin_amdgcn_exp2f((V[j] - lse) * kLog2e);
  } else {
    // Fig. 12: softmax over the k selected logits, max subtracted
    float denom = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      wgt[j] = (j < k) ? __builtin_amdgcn_exp2f((V[j] - V[0]) * kLog2e) : 0.f;
      denom += wgt[j];
    }
    const float inv = 1.f / denom;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) wgt[j] *= inv;
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k) stg[S::kGate + o + j] = wgt[j];
  if (want_logit) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) stg[S::kLogit + o + j] = V[j];
  }
  if (LSE) stg[S::kLse + lane] = lse;
}

// Bounded wait for an LDS word to reach `need` (sets abort on timeout or when
// another wave has aborted).
__device__ __forceinline__ bool sw_wait_ge(flag_ptr f, int need, flag_ptr abort_word, int limit) {
  return pc_wait(f, need, abort_word, limit);
}

template <int KMAX, int R16, bool LSE, bool FULL, int NC, int RING, int CAP>
__global__ __launch_bounds__(64 * (NC + 1)) void sweep_kernel(SweepArgs a) {
  typedef SwLds<R16, NC, RING, CAP, KMAX> L;
  typedef TpStage<KMAX> S;
  extern __shared__ __align__(16) char sw_lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x, w = blockIdx.x;
  const int NT = a.NT;
  const int P = min(max(__builtin_amdgcn_readfirstlane(__float_as_int(a.wstat[2])), 1), NT);
  const int Lseq = P + NT;
  if (threadIdx.x < 64) ((int*)sw_lds)[threadIdx.x] = 0;
  __syncthreads();
  flag_ptr fl = pc_flags(sw_lds);
  flag_ptr published = fl + L::kPub, prog = fl + L::kProg, abort_word = fl + L::kAbort;
  // rounds: consumer c of workgroup w routes blocks (round G + w) NC + c
  const long long per_round = (long long)G * NC;
  const int rounds = a.NB > (long long)w * NC ? (int)((a.NB - (long long)w * NC + per_round - 1) / per_round) : 0;

  if (wave == NC) {
    // ---------------------------------------------------------------- loader
    constexpr int LEAD = 4;          // tiles whose copies may still be in flight
    constexpr int DPT = R16 + 1;     // copies per tile
    const int total = rounds * Lseq;
    const rsrc_t r2d = make_rsrc(a.R2p, NT * R16 * 1024);
    const rsrc_t bqd = make_rsrc(a.biasq, NT * 256);
    int jseq = 0, slot_i = 0;   // g % Lseq and g % RING, kept incrementally
    int freed = 0;              // every consumer has read the tiles below this one
    for (int g = 0; g < total; ++g) {
      if (g - RING >= freed) {
        // slot g % RING is free once every consumer has read tile g - RING
        for (int it = 0;; ++it) {
          int mn = 0x7fffffff;
#pragma unroll
          for (int c = 0; c < NC; ++c) mn = min(mn, __builtin_amdgcn_readfirstlane(prog[c]));
          freed = mn;
          if (g - RING < freed) break;
          if (__builtin_amdgcn_readfirstlane(*abort_word) != 0 || it >= a.spin_limit) {
            *abort_word = 1;
            sw_fail(a.status, 1);
            return;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
      }
      const int t = jseq < P ? jseq : jseq - P;
      char* slot = sw_lds + L::kRing + slot_i * L::TB;
#pragma unroll
      for (int m = 0; m < R16; ++m)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r2d, (lds_void*)(slot + m * 1024), 16, lane * 16,
                                                 (t * R16 + m) * 1024, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(bqd, (lds_void*)(slot + R16 * 1024), 4, lane * 4, t * 256, 0, 0);
      if (g >= LEAD) {
        // the copies of tile g - LEAD (and older) have landed
        wait_vmcnt<LEAD * DPT>();
        asm volatile("" ::: "memory");
        *published = g - LEAD + 1;
      }
      if (++jseq == Lseq) jseq = 0;
      if (++slot_i == RING) slot_i = 0;
    }
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    *published = total;
    return;
  }

  // ---------------------------------------------------------------- consumer
  const int c = wave;
  const bool hi = lane >= 32;
  const int hf = hi ? 1 : 0;
  char* cl = sw_lds + L::kCons + c * L::kConsBytes;
  const SwLog lg{(lds_f4*)(cl + L::kLogV), (lds_u16*)(cl + L::kLogP)};
  lds_f32* stg = (lds_f32*)(cl + L::kStage);
  const float r2max = a.wstat[0], babs = a.wstat[1];
  // the seed tiles' smallest biases: lane t holds tile t's (read with v_readlane;
  // a per-tile vector load would wait on the whole vector-memory counter)
  const float bmv = lane < NT ? a.bmin[lane] : -__builtin_inff();
  // the ones operand of the bias MFMA: K slots 0 and 1 of every token column
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)((!hi && e < 2) ? 1.f : 0.f);
  floatx16 zero;
#pragma unroll
  for (int v = 0; v < 16; ++v) zero[v] = 0.f;

  auto zload = [&](long long b, bf16x8 (&h)[R16], bf16x8 (&l)[R16]) {
    const rsrc_t zd = make_rsrc((const char*)a.Z + (size_t)b * (2 * R16 * 1024), 2 * R16 * 1024);
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      h[m] = buf_load(zd, lane * 16 + m * 1024, 0);
      l[m] = buf_load(zd, lane * 16 + (R16 + m) * 1024, 0);
    }
  };
  bf16x8 zh[R16], zl[R16], nh[R16], nl[R16];
  if (rounds > 0) zload((long long)w * NC + c, nh, nl);
  bool ok = true;
  int pub = 0;   // tiles known to be published
  for (int round = 0; round < rounds && ok; ++round) {
    const long long b = ((long long)round * G + w) * NC + c;
    if (b >= a.NB) break;
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      zh[m] = nh[m];
      zl[m] = nl[m];
    }
    if (b + per_round < a.NB) zload(b + per_round, nh, nl);
    // eps of the token (both lanes hold half of z each)
    float sl = 0.f, sh = 0.f;
#pragma unroll
    for (int m = 0; m < R16; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float u = (float)zl[m][e], v = (float)zh[m][e];
        sl = __builtin_fmaf(u, u, sl);
        sh = __builtin_fmaf(v, v, sh);
      }
    sl += partner_f32(sl, hi);
    sh += partner_f32(sh, hi);
    const float eps = __builtin_sqrtf(sl) * r2max + 0x1p-15f * (__builtin_sqrtf(sh) * r2max + babs);

    TwoPassState<KMAX> st;
    st.init(a.k);
    const int g0 = round * Lseq;
    // two operand buffers and two accumulators, used alternately (the buffer
    // index is a compile-time constant in each half of the loop body)
    bf16x8 opA[R16], opB[R16];
    uint32_t bqA = 0, bqB = 0;
    floatx16 accA, accB;
    // tile j's operands -> (op, bq), once the loader has published it (the
    // published count is polled only when the cached one runs out)
    auto fetch = [&](int j, bf16x8 (&op)[R16], uint32_t& bq) -> bool {
      const int g = g0 + j;
      if (g >= pub) {
        if (!sw_wait_ge(published, g + 1, abort_word, a.spin_limit)) return false;
        pub = __builtin_amdgcn_readfirstlane(*published);
        asm volatile("" ::: "memory");
      }
      lds_cchar* slot = (lds_cchar*)(sw_lds + L::kRing + (g % RING) * L::TB);
#pragma unroll
      for (int m = 0; m < R16; ++m) op[m] = *(lds_cbf16x8*)(slot + m * 1024 + lane * 16);
      bq = *(lds_cu32*)(slot + R16 * 1024 + lane * 4);
      return true;
    };
    // the MFMAs of tile j
    auto mfmas = [&](int j, const bf16x8 (&op)[R16], uint32_t bq) -> floatx16 {
      floatx16 acc;
      if (j < P) {
        acc = mfma_bf16(op[0], zh[0], zero);
#pragma unroll
        for (int m = 1; m < R16; ++m) acc = mfma_bf16(op[m], zh[m], acc);
      } else {
        const bf16x8 bop = __builtin_bit_cast(bf16x8, u32x4{bq, 0u, 0u, 0u});
        acc = mfma_bf16(bop, ones, zero);
#pragma unroll
        for (int m = 0; m < R16; ++m) acc = mfma_bf16(op[m], zh[m], acc);
#pragma unroll
        for (int m = 0; m < R16; ++m) acc = mfma_bf16(op[m], zl[m], acc);
      }
      return acc;
    };
    // the VALU side of tile j (its accumulator holds the logits)
    auto valu = [&](int j, const floatx16& acc_j) {
      if (j < P) {
        // seed: the tile maximum plus the tile's smallest bias is at most
        // (up to eps) the logit of one real expert
        const float bm = j < kWave ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bmv), j)) : a.bmin[j];
        const float lb = max16(acc_j) + bm;
        med3_insert<KMAX>(st.L, lb);
      } else {
        const int t = j - P;
        if (LSE) {
          floatx4 gq;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            gq[q] = fmaxf(fmaxf(acc_j[4 * q], acc_j[4 * q + 1]), fmaxf(acc_j[4 * q + 2], acc_j[4 * q + 3]));
          tp_lse_tile<KMAX>(st, acc_j, gq);
        }
        sw_log_tile<KMAX, CAP>(st, acc_j, kTile * t + 4 * hf, lg, lane, hi, a.k, a.perm);
        if (t == kTightenTile - 1 && NT > kTightenTile) {
          const float2 r = sw_tighten<KMAX, CAP>(st.thr, st.cnt, lg, lane, hi, a.k, a.perm);
          st.thr = r.x;
          st.cnt = __float_as_int(r.y);
        }
      }
      if (j == P - 1) {
        // end of the seed: the token's threshold
        tp_threshold<KMAX>(st, hi, a.k);
        st.thr -= eps;
      }
    };
    // tile j has been read once its MFMAs are issued: the asm makes its operand
    // registers (hence the LDS reads) complete before the progress word moves
    auto consumed = [&](int j, const bf16x8 (&op)[R16], uint32_t bq) {
#pragma unroll
      for (int m = 0; m < R16; ++m) asm volatile("" ::"v"(op[m]));
      asm volatile("" ::"v"(bq) : "memory");
      prog[c] = g0 + j + 1;
    };
    // software pipeline: the MFMAs of tile j run while the VALU works on tile j - 1
    ok = fetch(0, opA, bqA);
    int j = 0;
    for (; j + 1 < Lseq && ok; j += 2) {
      ok = fetch(j + 1, opB, bqB);
      if (!ok) break;
      accA = mfmas(j, opA, bqA);
      consumed(j, opA, bqA);
      if (j >= 1) valu(j - 1, accB);
      if (j + 2 < Lseq) {
        ok = fetch(j + 2, opA, bqA);
        if (!ok) break;
      }
      accB = mfmas(j + 1, opB, bqB);
      consumed(j + 1, opB, bqB);
      valu(j, accA);
    }
    if (!ok) break;
    // tail: Lseq odd leaves tile Lseq - 1 (its operands are in opA)
    if (j < Lseq) {
      accA = mfmas(j, opA, bqA);
      consumed(j, opA, bqA);
      if (j >= 1) valu(j - 1, accB);
      valu(j, accA);
    } else {
      valu(Lseq - 1, accB);
    }

    // finish: results (sweep positions in the idx words) into the result block
    sw_finish<KMAX, FULL, LSE>(st, lg, lane, hi, a.perm, a.k, a.out_logit != nullptr, stg);
    lds_drain();
    // sweep positions -> expert indices (lanes 0..31, one token each)
    if (!hi) {
      int pidx[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < a.k) {
          const int p = __float_as_int(stg[S::kIdx + lane * a.k + j]);
          pidx[j] = a.perm[min(max(p, 0), NT * kTile - 1)];
        }
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < a.k) stg[S::kIdx + lane * a.k + j] = __int_as_float(pidx[j]);
    }
    lds_drain();
    // result block -> memory: one 16-byte store per lane and array; the
    // descriptor range drops the rows past N
    const long long n0 = b * kTile;
    const long long rows = a.N - n0 < kTile ? a.N - n0 : kTile;
    const int bk = (int)rows * a.k * 4;
    lds_cchar* sb = (lds_cchar*)stg;
    const u32x4 vi = lds_ld128(sb, S::kIdx * 4 + lane * 16);
    const u32x4 vg = lds_ld128(sb, S::kGate * 4 + lane * 16);
    __builtin_amdgcn_raw_buffer_store_b128(vi, make_rsrc(a.out_idx + n0 * a.k, bk), lane * 16, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(vg, make_rsrc(a.out_gate + n0 * a.k, bk), lane * 16, 0, 0);
    if (KMAX > 8) {
      // 32 k words per array may exceed one 16-byte store per lane
      const u32x4 vi2 = lds_ld128(sb, S::kIdx * 4 + 1024 + lane * 16);
      const u32x4 vg2 = lds_ld128(sb, S::kGate * 4 + 1024 + lane * 16);
      __builtin_amdgcn_raw_buffer_store_b128(vi2, make_rsrc(a.out_idx + n0 * a.k, bk), 1024 + lane * 16, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(vg2, make_rsrc(a.out_gate + n0 * a.k, bk), 1024 + lane * 16, 0, 0);
    }
    if (a.out_logit) {
      const u32x4 vl = lds_ld128(sb, S::kLogit * 4 + lane * 16);
      __builtin_amdgcn_raw_buffer_store_b128(vl, make_rsrc(a.out_logit + n0 * a.k, bk), lane * 16, 0, 0);
      if (KMAX > 8) {
        const u32x4 vl2 = lds_ld128(sb, S::kLogit * 4 + 1024 + lane * 16);
        __builtin_amdgcn_raw_buffer_store_b128(vl2, make_rsrc(a.out_logit + n0 * a.k, bk), 1024 + lane * 16, 0, 0);
      }
    }
    if (LSE && a.out_lse) {
      const u32x4 vz = lds_ld128(sb, S::kLse * 4 + lane * 16);
      __builtin_amdgcn_raw_buffer_store_b128(vz, make_rsrc(a.out_lse + n0, (int)rows * 4), lane * 16, 0, 0);
    }
    // the result block is rewritten by the next finish only after these reads
    lds_drain();
  }
  if (!ok) sw_fail(a.status, 1);
  // retire: the loader no longer waits for this consumer
  asm volatile("" ::: "memory");
  prog[c] = 0x7fffffff;
}

}  // namespace more
