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
// Exact top-k per token (ties to the lower expert index).  Every tile's
// logits are exact (bias included): the bias as a bf16 hi + lo operand
// against a ones operand, then z_hi and z_lo against the tile's R2 operands
// (2 R16 + 1 MFMAs, fp32 accumulation).
//   seed pass (the first P tiles of the sweep order -- bias descending, so
//     they hold most winners -- or every tile without a bias): each lane keeps
//     the k largest of its tile maxima (v_med3 list); a tile maximum is the
//     logit of one expert, so the k-th largest over the token's two lanes,
//     thr, is at most its k-th logit.
//   main sweep (every tile): a 4-logit group whose maximum reaches thr is
//     appended to the lane's log (16 bytes + a 16-bit sweep position).  Every
//     top-k logit is >= thr, so it is logged.  When some lane's appends would
//     not fit -- and once after the first kTightenTile main tiles, where the
//     high-bias winners are -- the whole wave tightens: thr rises to the
//     token's k-th largest logged group maximum (each is the logit of a
//     distinct expert, so still a lower bound of the k-th logit) and groups
//     below it are dropped.
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
  const int* seed;           // seed tiles P (1 <= P <= NT): written by the packing call
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

// Loader waves per workgroup: loader i copies the sequence tiles g = i (mod
// kSwLoaders), so that the copies of several tiles are issued at once.
constexpr int kSwLoaders = 2;

// LDS map.  Flag words (ints): published[kSwLoaders] (loader i has copied its
// tiles below published[i]; tile g sits in slot g % RING), prog[NC] (tiles
// each consumer has finished reading), abort.
template <int R16, int NC, int RING, int CAP, int KMAX>
struct SwLds {
  static constexpr int TB = R16 * 1024 + 256;   // ring slot: R16 A operands + 64 bias words
  static constexpr int kPub = 0, kProg = kSwLoaders, kAbort = kSwLoaders + NC;
  static_assert(NC + kSwLoaders + 1 <= 64, "flag words");
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

// Per-group appends with a capacity check before each (out of line: taken
// when a lane's log is nearly full even after a tightening, i.e. with many
// exact ties).  Whole wave active; returns (thr, count as int bits).
template <int KMAX, int CAP>
__device__ __noinline__ float2 sw_log_slow(floatx16 acc, float thr, int cnt, int pos_base, SwLog lg, int lane,
                                           bool hi_half, int k, const int* __restrict__ perm) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float g = fmaxf(fmaxf(acc[4 * q], acc[4 * q + 1]), fmaxf(acc[4 * q + 2], acc[4 * q + 3]));
    if (any_lane(g >= thr)) {
      if (any_lane(cnt >= CAP)) {
        const float2 r = sw_tighten<KMAX, CAP>(thr, cnt, lg, lane, hi_half, k, perm);
        thr = r.x;
        cnt = __float_as_int(r.y);
      }
      if (g >= thr) {
        lg.val[cnt * kWave + lane] = floatx4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        lg.pos[cnt * kWave + lane] = (uint16_t)(pos_base + 8 * q);
        ++cnt;
      }
    }
  }
  return make_float2(thr, __int_as_float(cnt));
}

// Main-sweep logging of one tile (acc: this lane's 16 exact logits, bias
// included, -inf on padding rows; gq: the maxima of its four 4-logit groups;
// pos_base = 32 t + 4 hf; register 4q + e is sweep row 8q + 4hf + e).  A lane
// appends each of its groups whose maximum reaches thr (16 bytes + the 16-bit
// sweep position of the group's first logit).
template <int KMAX, int CAP>
__device__ __forceinline__ void sw_log_tile(TwoPassState<KMAX>& st, const floatx16& acc, const floatx4& gq,
                                            int pos_base, SwLog lg, int lane, bool hi_half, int k,
                                            const int* __restrict__ perm) {
  const float tmax = fmaxf(fmaxf(gq[0], gq[1]), fmaxf(gq[2], gq[3]));
  if (!any_lane(tmax >= st.thr)) return;
  auto hits = [&]() {
    int n = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) n += gq[q] >= st.thr ? 1 : 0;
    return n;
  };
  // The appends below write slot cnt in every lane (a lane without a hit
  // writes its next free slot, which stays free), so cnt + hits must stay
  // below CAP: the last slot is the spare of a full lane.
  if (any_lane(st.cnt > CAP - 5) && any_lane(st.cnt + hits() > CAP - 1)) {
    // some lane's appends would not fit: tighten first
    const float2 r = sw_tighten<KMAX, CAP>(st.thr, st.cnt, lg, lane, hi_half, k, perm);
    st.thr = r.x;
    st.cnt = __float_as_int(r.y);
    if (any_lane(st.cnt + hits() > CAP - 1)) {
      const float2 r2 = sw_log_slow<KMAX, CAP>(acc, st.thr, st.cnt, pos_base, lg, lane, hi_half, k, perm);
      st.thr = r2.x;
      st.cnt = __float_as_int(r2.y);
      return;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    lg.val[st.cnt * kWave + lane] = floatx4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    lg.pos[st.cnt * kWave + lane] = (uint16_t)(pos_base + 8 * q);
    st.cnt += gq[q] >= st.thr ? 1 : 0;
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
__global__ __launch_bounds__(64 * (NC + kSwLoaders)) void sweep_kernel(SweepArgs a) {
  typedef SwLds<R16, NC, RING, CAP, KMAX> L;
  typedef TpStage<KMAX> S;
  extern __shared__ __align__(16) char sw_lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x, w = blockIdx.x;
  const int NT = a.NT;
  // seed tiles, even (NT is even: the expert count is padded to a multiple of 64)
  const int P = min((max(__builtin_amdgcn_readfirstlane(*a.seed), 1) + 1) & ~1, NT);
  const int Lseq = P + NT;
  if (threadIdx.x < 64) ((int*)sw_lds)[threadIdx.x] = 0;
  __syncthreads();
  flag_ptr fl = pc_flags(sw_lds);
  flag_ptr published = fl + L::kPub, prog = fl + L::kProg, abort_word = fl + L::kAbort;
  // rounds: consumer c of workgroup w routes blocks (round G + w) NC + c
  const long long per_round = (long long)G * NC;
  const int rounds = a.NB > (long long)w * NC ? (int)((a.NB - (long long)w * NC + per_round - 1) / per_round) : 0;

  if (wave >= NC) {
    // ---------------------------------------------------------------- loaders
    // own tiles whose copies may still be in flight; the ring must hold them
    // plus the two tiles a consumer reads ahead (no circular wait)
    constexpr int LEAD = RING / kSwLoaders - 2 < 4 ? RING / kSwLoaders - 2 : 4;
    constexpr int DPT = R16 + 1;     // copies per tile
    static_assert(LEAD >= 1 && RING >= kSwLoaders * (LEAD + 1) + 1, "ring depth");
    const int li = wave - NC;
    const int total = rounds * Lseq;
    const rsrc_t r2d = make_rsrc(a.R2p, NT * R16 * 1024);
    const rsrc_t bqd = make_rsrc(a.biasq, NT * 256);
    int jseq = li, slot_i = li;   // g % Lseq and g % RING, kept incrementally
    int freed = 0;                // every consumer has read the tiles below this one
    int n = 0;                    // own tiles issued
    for (int g = li; g < total; g += kSwLoaders, ++n) {
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
      if (n >= LEAD) {
        // the copies of own tile g - LEAD * kSwLoaders (and older) have landed
        wait_vmcnt<LEAD * DPT>();
        asm volatile("" ::: "memory");
        published[li] = g - LEAD * kSwLoaders + 1;
      }
      jseq += kSwLoaders;
      if (jseq >= Lseq) jseq -= Lseq;
      slot_i += kSwLoaders;
      if (slot_i >= RING) slot_i -= RING;
    }
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    published[li] = total;
    return;
  }

  // ---------------------------------------------------------------- consumer
  const int c = wave;
  const bool hi = lane >= 32;
  const int hf = hi ? 1 : 0;
  char* cl = sw_lds + L::kCons + c * L::kConsBytes;
  const SwLog lg{(lds_f4*)(cl + L::kLogV), (lds_u16*)(cl + L::kLogP)};
  lds_f32* stg = (lds_f32*)(cl + L::kStage);
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
  const int total = rounds * Lseq;   // the loader's sequence
  int pub = 0;                       // tiles known to be published
  bool stalled = false;              // a bounded wait gave up (results are void)
  // sequence tile g's operands -> (op, bq).  Reads past the sequence end
  // re-read its last tile (the prefetch of a round that does not follow).
  auto fetch = [&](int g, bf16x8 (&op)[R16], uint32_t& bq) {
    g = min(g, total - 1);
    if (g >= pub) {
      // every tile below the smallest published count is in the ring
      for (int it = 0;; ++it) {
        int mn = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kSwLoaders; ++i) mn = min(mn, __builtin_amdgcn_readfirstlane(published[i]));
        pub = mn;
        if (g < pub) break;
        if (__builtin_amdgcn_readfirstlane(*abort_word) != 0 || it >= a.spin_limit) {
          *abort_word = 1;
          stalled = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      asm volatile("" ::: "memory");
    }
    lds_cchar* slot = (lds_cchar*)(sw_lds + L::kRing + ((unsigned)g % RING) * L::TB);
#pragma unroll
    for (int m = 0; m < R16; ++m) op[m] = *(lds_cbf16x8*)(slot + m * 1024 + lane * 16);
    bq = *(lds_cu32*)(slot + R16 * 1024 + lane * 4);
  };
  // tile g has been read once its MFMAs are issued: the asm makes the operand
  // registers (hence the LDS reads) complete before the progress word moves
  auto consumed = [&](int g, const bf16x8 (&op)[R16], uint32_t bq) {
#pragma unroll
    for (int m = 0; m < R16; ++m) asm volatile("" ::"v"(op[m]));
    asm volatile("" ::"v"(bq) : "memory");
    prog[c] = g + 1;
  };

  bf16x8 zh[R16], zl[R16], nh[R16], nl[R16];
  bf16x8 opA[R16], opB[R16];
  uint32_t bqA = 0, bqB = 0;
  if (rounds > 0) {
    zload((long long)w * NC + c, nh, nl);
    fetch(0, opA, bqA);
    fetch(1, opB, bqB);
  }
  for (int round = 0; round < rounds && !stalled; ++round) {
    const long long b = ((long long)round * G + w) * NC + c;
    if (b >= a.NB) break;
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      zh[m] = nh[m];
      zl[m] = nl[m];
    }
    if (b + per_round < a.NB) zload(b + per_round, nh, nl);
    // exact logits of one tile: the bias (hi + lo against the ones operand),
    // then z_hi and z_lo against the tile's R2 operands
    auto mfmas = [&](const bf16x8 (&op)[R16], uint32_t bq) -> floatx16 {
      const bf16x8 bop = __builtin_bit_cast(bf16x8, u32x4{bq, 0u, 0u, 0u});
      floatx16 acc = mfma_bf16(bop, ones, zero);
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(op[m], zh[m], acc);
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(op[m], zl[m], acc);
      return acc;
    };
    TwoPassState<KMAX> st;
    st.init(a.k);
    const int g0 = round * Lseq;
    // seed: the lane's tile maximum is the exact logit of one expert; the k
    // largest of these over both lanes bound the token's k-th logit from below
    auto seed = [&](const floatx16& acc) { med3_insert<KMAX>(st.L, max16(acc)); };
    // main-sweep tile, straight-line part: group maxima and the running normaliser
    auto pre = [&](const floatx16& acc) -> floatx4 {
      floatx4 gq;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        gq[q] = fmaxf(fmaxf(acc[4 * q], acc[4 * q + 1]), fmaxf(acc[4 * q + 2], acc[4 * q + 3]));
      if (LSE) tp_lse_tile<KMAX>(st, acc, gq);
      return gq;
    };
    // main-sweep tile t, branching part: the appends, and the scheduled tightening
    auto post = [&](const floatx16& acc, const floatx4& gq, int t) {
      sw_log_tile<KMAX, CAP>(st, acc, gq, kTile * t + 4 * hf, lg, lane, hi, a.k, a.perm);
      if (t == kTightenTile - 1 && NT > kTightenTile) {
        const float2 r = sw_tighten<KMAX, CAP>(st.thr, st.cnt, lg, lane, hi, a.k, a.perm);
        st.thr = r.x;
        st.cnt = __float_as_int(r.y);
      }
    };
    // Interleave the MFMAs of one tile with the straight-line VALU work of the
    // previous one in the instruction stream (the wave issues VALU work while
    // its MFMAs occupy the matrix pipe).
    auto interleave = [&]() {
#pragma unroll
      for (int i = 0; i < 2 * R16 + 1; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
    };
    // keep a value's computation in front of this point (the compiler would
    // otherwise sink it past the polls, away from the MFMAs it should overlap)
    auto pin_seed = [&]() {
#pragma unroll
      for (int i = 0; i < KMAX; ++i) asm volatile("" ::"v"(st.L[i]));
    };
    auto pin4 = [&](const floatx4& v) { asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3])); };
    // Software pipeline: the MFMAs of the next tile are issued with the VALU
    // work of the current one.  Entering: opA / opB hold sequence tiles g0 and
    // g0 + 1 (P and Lseq are even).
    floatx16 accA, accB;
    accA = mfmas(opA, bqA);
    consumed(g0, opA, bqA);
    fetch(g0 + 2, opA, bqA);
    for (int j = 0; j < P; j += 2) {
      accB = mfmas(opB, bqB);
      seed(accA);
      interleave();
      pin_seed();
      consumed(g0 + j + 1, opB, bqB);
      fetch(g0 + j + 3, opB, bqB);
      accA = mfmas(opA, bqA);
      seed(accB);
      interleave();
      pin_seed();
      consumed(g0 + j + 2, opA, bqA);
      fetch(g0 + j + 4, opA, bqA);
    }
    tp_threshold<KMAX>(st, hi, a.k);
    // accA: sequence tile g0 + P (main tile 0) in flight
    for (int j = P; j < Lseq; j += 2) {
      accB = mfmas(opB, bqB);
      const floatx4 gA = pre(accA);
      interleave();
      pin4(gA);
      consumed(g0 + j + 1, opB, bqB);
      fetch(g0 + j + 3, opB, bqB);
      post(accA, gA, j - P);
      floatx4 gB;
      if (j + 2 < Lseq) {
        accA = mfmas(opA, bqA);
        gB = pre(accB);
        interleave();
        pin4(gB);
        consumed(g0 + j + 2, opA, bqA);
        fetch(g0 + j + 4, opA, bqA);
      } else {
        gB = pre(accB);
      }
      post(accB, gB, j + 1 - P);
    }
    // opA / opB now hold the next round's first two tiles
    if (stalled) break;

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
  if (stalled) sw_fail(a.status, 1);
  // retire: the loader no longer waits for this consumer
  asm volatile("" ::: "memory");
  prog[c] = 0x7fffffff;
}

}  // namespace more
