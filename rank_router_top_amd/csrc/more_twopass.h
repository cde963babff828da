// more_twopass.h -- two-pass exact top-k over the expert tiles of one token
// block, used by the producer/consumer kernel.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.1 Algorithm 1 (one sweep over the experts with a running
// top-k buffer; logits never leave the chip) and App. F.2.1 eq. (8) (running
// maximum and normaliser for the full-softmax gate).  The selected set is the
// exact top-k (ties to the lower expert index); only the way it is found
// differs from a single running buffer.
//
// Why two passes on gfx950: a token's 32 logits of a tile are spread over two
// lanes (16 each), and the 64 lanes of a wave move in lockstep.  With one
// running buffer the threshold is far below its final value for the first
// tens of tiles, candidates are scattered over lanes and positions, and every
// wave-level insertion does useful work in only a few lanes.  Recomputing the
// logits is cheap in comparison (4 MFMAs per tile), so:
//
//   pass 1 (branch-free): per lane, a v_med3 list of the k largest TILE MAXIMA
//     (16 VALU per tile); at the end the two halves of a token merge their
//     lists, and the token threshold thr = k-th largest of all half-tile
//     maxima.  Each of those maxima is a distinct logit, so at least k logits
//     are >= thr: thr is a lower bound of the token's k-th logit (and equal to
//     it whenever no two of the top k share a half-tile).  The full-softmax
//     normaliser (eq. 8) is accumulated here too (pass 1 then covers all tiles).
//   pass 2: recompute each tile; only lanes with a logit >= thr do anything:
//     they append (logit, sweep position) to their LDS log.  Every logit of
//     the final top-k is >= thr, so it is in one of the token's two logs.
//   seeded form: with a bias, pass 1 runs over the first tiles of the
//     bias-descending order only (they hold most of the winners), and pass 2
//     keeps raising thr with the maxima of the other tiles (tp_pass2_tile).
//   finish: merge the two logs by (logit desc, expert index asc).
//
// If a log fills up (odd shapes, massive exact ties), it is compacted: the
// lane's own k-th largest logged value raises its threshold (still a lower
// bound of the token's k-th), entries below are dropped, and among exact ties
// at the threshold only the k of lowest expert index are kept.
#pragma once
#include "more_device.h"

namespace more {

template <int KMAX>
struct TwoPassState {
  float L[KMAX];   // pass 1: descending; the first KMAX-k slots hold +inf (runtime k < KMAX)
  float thr;       // pass 2 threshold of this lane
  int cnt;         // pass 2 log entries of this lane
  float m, Z;      // running maximum / normaliser (full-softmax gate)

  __device__ __forceinline__ void init(int k) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) L[j] = (j < KMAX - k) ? __builtin_inff() : kLowest;
    thr = kLowest;
    cnt = 0;
    m = kLowest * 0.25f;
    Z = 0.f;
  }
};

template <int KMAX>
__device__ __forceinline__ void med3_insert(float (&L)[KMAX], float x) {
#pragma unroll
  for (int j = KMAX - 1; j >= 1; --j) L[j] = __builtin_amdgcn_fmed3f(L[j - 1], L[j], x);
  L[0] = fmaxf(L[0], x);
}

__device__ __forceinline__ float max16(const floatx16& a) {
  const float g0 = fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
  const float g1 = fmaxf(fmaxf(a[4], a[5]), fmaxf(a[6], a[7]));
  const float g2 = fmaxf(fmaxf(a[8], a[9]), fmaxf(a[10], a[11]));
  const float g3 = fmaxf(fmaxf(a[12], a[13]), fmaxf(a[14], a[15]));
  return fmaxf(fmaxf(g0, g1), fmaxf(g2, g3));
}

// Pass 1, one tile (acc: this lane's 16 logits of the tile, -inf on padding).
template <int KMAX, bool FULL>
__device__ __forceinline__ void tp_pass1_tile(TwoPassState<KMAX>& st, const floatx16& acc) {
  const float tmax = max16(acc);
  if (FULL) {
    // eq. (8): rescale the running sum when the maximum moves, then add the tile
    const float mn = fmaxf(st.m, tmax);
    const float mb = mn * kLog2e;
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) s += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], kLog2e, -mb));
    st.Z = st.Z * __builtin_amdgcn_exp2f((st.m - mn) * kLog2e) + s;
    st.m = mn;
  }
  med3_insert<KMAX>(st.L, tmax);
}

// Pass 1 with the four group maxima of the tile instead of its maximum: the
// groups are disjoint, so their maxima are distinct logits of the token and
// the k-th largest of them is still a lower bound of its k-th logit, a much
// closer one when a lane sees few tiles (the expert shards of the split-M
// form).  16 more VALU per tile and list length.
template <int KMAX>
__device__ __forceinline__ void tp_pass1_groups(TwoPassState<KMAX>& st, const floatx16& acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    med3_insert<KMAX>(st.L, fmaxf(fmaxf(acc[4 * q], acc[4 * q + 1]), fmaxf(acc[4 * q + 2], acc[4 * q + 3])));
}

// End of pass 1: token threshold = k-th largest of both halves' tile maxima
// (identical on the two lanes of a token).
template <int KMAX>
__device__ __forceinline__ void tp_threshold(TwoPassState<KMAX>& st, bool hi_half, int k) {
  float T[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) T[j] = st.L[j];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const float p = partner_f32(st.L[j], hi_half);
    med3_insert<KMAX>(T, j >= KMAX - k ? p : kLowest);   // the partner's +inf pads are skipped
  }
  st.thr = T[KMAX - 1];
  st.cnt = 0;
}

// Out of line (rare): raise thr to the lane's own k-th largest logged value,
// then drop entries below it (and surplus exact ties, by expert index).
// Returns (new thr, new count as int bits).  Called with the whole wave active.
template <int KMAX, class PT>
__device__ __noinline__ float2 tp_compact(float2* base, int lane, int cnt, float thr, PT perm, int k, int cap) {
  float L[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) L[j] = (j < KMAX - k) ? __builtin_inff() : kLowest;
  for (int c = 0; c < cnt; ++c) med3_insert<KMAX>(L, base[c * kWave + lane].x);
  const float t2 = fmaxf(thr, L[KMAX - 1]);
  return make_float2(t2, __int_as_float(compact_log(base, lane, cnt, t2, perm, k, cap)));
}

// Pass 2, one tile: append every logit >= thr with its sweep position
// (pos_base = 32 t + 4 hf; register v of the lane is row 8(v/4) + 4hf + v%4).
// Inside a group of 4 rows that holds a candidate in some lane the appends
// are branch-free: each value is written to slot cnt and cnt advances only if
// it qualifies.  Needs cnt <= CAP - 4 before a group (compacted otherwise).
//
// Seeded form (RUN): pass 1 ran over the first tiles of the bias-descending
// order only, so this pass is the one full sweep.  A tile outside the seed
// (run) adds its maximum to the lane's list of half-tile maxima and raises thr
// to the list's k-th entry (distinct logits of the token: still a lower bound
// of its k-th) before its appends.
// The branch-free part of a pass-2 tile: group maxima (4 rows each) and, in
// the seeded form, the insertion of the tile maximum (x = -inf when the tile
// was part of the seed: a no-op) and the raise of thr.
template <int KMAX, bool RUN>
__device__ __forceinline__ floatx4 tp_pass2_scan(TwoPassState<KMAX>& st, const floatx16& acc, bool run) {
  floatx4 g;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    g[q] = fmaxf(fmaxf(acc[4 * q], acc[4 * q + 1]), fmaxf(acc[4 * q + 2], acc[4 * q + 3]));
  if (RUN) {
    const float tmax = fmaxf(fmaxf(g[0], g[1]), fmaxf(g[2], g[3]));
    med3_insert<KMAX>(st.L, run ? tmax : -__builtin_inff());
    st.thr = fmaxf(st.thr, st.L[KMAX - 1]);
  }
  return g;
}

// eq. (8) over one pass-2 tile (group maxima g from tp_pass2_scan): rescale
// the running sum when the maximum moves, then add the tile.
template <int KMAX>
__device__ __forceinline__ void tp_lse_tile(TwoPassState<KMAX>& st, const floatx16& acc, const floatx4& g) {
  const float tmax = fmaxf(fmaxf(g[0], g[1]), fmaxf(g[2], g[3]));
  const float mn = fmaxf(st.m, tmax);
  const float mb = mn * kLog2e;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int v = 0; v < 16; v += 2) {
    s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], kLog2e, -mb));
    s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v + 1], kLog2e, -mb));
  }
  st.Z = st.Z * __builtin_amdgcn_exp2f((st.m - mn) * kLog2e) + (s0 + s1);
  st.m = mn;
}

// The appends of a pass-2 tile (group maxima g from tp_pass2_scan).
template <int KMAX, int CAP, class PT>
__device__ __forceinline__ void tp_pass2_log(TwoPassState<KMAX>& st, const floatx16& acc, const floatx4& g,
                                             int pos_base, LogRef lg, int lane, PT perm, int k) {
  const float tmax = fmaxf(fmaxf(g[0], g[1]), fmaxf(g[2], g[3]));
  if (any_lane(tmax >= st.thr)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (any_lane(g[q] >= st.thr)) {
        if (any_lane(st.cnt > CAP - 4)) {
          const float2 r = tp_compact<KMAX>(lg.base, lane, st.cnt, st.thr, perm, k, CAP);
          st.thr = r.x;
          st.cnt = __float_as_int(r.y);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = acc[4 * q + e];
          lg.base[st.cnt * kWave + lane] = make_float2(x, __int_as_float(pos_base + 8 * q + e));
          st.cnt += (x >= st.thr) ? 1 : 0;
        }
      }
    }
    lds_drain();   // as in tp_pass2_groups: keep the LDS counter uniform after the branch
  }
}

template <int KMAX, int CAP, bool RUN, class PT>
__device__ __forceinline__ void tp_pass2_tile(TwoPassState<KMAX>& st, const floatx16& acc, bool run, int pos_base,
                                              LogRef lg, int lane, PT perm, int k) {
  const floatx4 g = tp_pass2_scan<KMAX, RUN>(st, acc, run);
  tp_pass2_log<KMAX, CAP>(st, acc, g, pos_base, lg, lane, perm, k);
}

// ---------------------------------------------------------------- group log
// Pass 2 with a log of 4-logit groups instead of single logits.  A group is
// the 4 consecutive accumulator registers 4q..4q+3 of a lane (rows 8q+4hf ..
// +3 of the tile, sweep positions gpos .. gpos+3): when its maximum reaches
// thr, the lane appends the whole group with one 16-byte LDS store plus its
// position, and the wave spends ~5 instructions on it instead of ~28 for four
// branch-free single-logit appends.  Logits below thr inside a logged group
// are dropped at the finish.
struct GroupLog {
  lds_f4* val;    // entry c of lane l: val[c * 64 + l] (the 4 logits)
  lds_i32* pos;   // pos[c * 64 + l]: sweep position of the group's first logit
};

// Out of line (rare: the lane's log is full): raise thr to the lane's own
// k-th largest logged logit (a lower bound of the token's k-th), drop groups
// whose maximum is below it, and where exact ties at that value would keep
// more than k groups, keep only the tied logits of lowest expert index (the
// others can never be selected).  Afterwards at most k groups remain.
// Returns (new thr, new count as int bits).  Called with the whole wave active.
template <int KMAX, class PT>
__device__ __noinline__ float2 tp_compact_groups(lds_f4* val, lds_i32* pos, int lane, int cnt, float thr, PT perm,
                                                 int k) {
  float L[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) L[j] = (j < KMAX - k) ? __builtin_inff() : kLowest;
  for (int c = 0; c < cnt; ++c) {
    const floatx4 v = val[c * kWave + lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) med3_insert<KMAX>(L, v[e]);
  }
  const float t2 = fmaxf(thr, L[KMAX - 1]);
  int w = 0, gt = 0;
  for (int c = 0; c < cnt; ++c) {
    const floatx4 v = val[c * kWave + lane];
    const float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
#pragma unroll
    for (int e = 0; e < 4; ++e) gt += v[e] > t2 ? 1 : 0;
    if (m >= t2) {
      const int p = pos[c * kWave + lane];
      val[w * kWave + lane] = v;
      pos[w * kWave + lane] = p;
      ++w;
    }
  }
  cnt = w;
  if (cnt > k) {
    // exact ties at t2: keep the (k - gt) of lowest expert index
    const int keep = k - gt;
    for (int c = 0; c < cnt; ++c) {
      floatx4 v = val[c * kWave + lane];
      const int p = pos[c * kWave + lane];
      bool changed = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (v[e] == t2) {
          const int oi = perm[p + e];
          int rank = 0;
          for (int c2 = 0; c2 < cnt; ++c2) {
            const floatx4 v2 = val[c2 * kWave + lane];
            const int p2 = pos[c2 * kWave + lane];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2)
              if (v2[e2] == t2 && (int)perm[p2 + e2] < oi) ++rank;
          }
          if (rank >= keep) {
            v[e] = -__builtin_inff();
            changed = true;
          }
        }
      }
      if (changed) val[c * kWave + lane] = v;
    }
    w = 0;
    for (int c = 0; c < cnt; ++c) {
      const floatx4 v = val[c * kWave + lane];
      if (fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])) >= t2) {
        const int p = pos[c * kWave + lane];
        val[w * kWave + lane] = v;
        pos[w * kWave + lane] = p;
        ++w;
      }
    }
    cnt = w;
  }
  return make_float2(t2, __int_as_float(cnt));
}

// Pass 2, the appends of one tile (group maxima g from tp_pass2_scan; pos_base
// = 32 t + 4 hf, register v of the lane is row 8(v/4) + 4hf + v%4).  Needs
// CAPG >= KMAX + 1 (a compaction leaves at most k groups).
template <int KMAX, int CAPG, class PT>
__device__ __forceinline__ void tp_pass2_groups(TwoPassState<KMAX>& st, const floatx16& acc, const floatx4& g,
                                                int pos_base, GroupLog lg, int lane, PT perm, int k) {
  static_assert(CAPG >= KMAX + 1, "a compacted log must leave room for one more group");
  const float tmax = fmaxf(fmaxf(g[0], g[1]), fmaxf(g[2], g[3]));
  if (any_lane(tmax >= st.thr)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool hit = g[q] >= st.thr;
      if (any_lane(hit)) {
        if (any_lane(st.cnt >= CAPG)) {
          const float2 r = tp_compact_groups<KMAX>(lg.val, lg.pos, lane, st.cnt, st.thr, perm, k);
          st.thr = r.x;
          st.cnt = __float_as_int(r.y);
        }
        // every lane writes its slot cnt; only a hit advances cnt
        lg.val[st.cnt * kWave + lane] = floatx4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        lg.pos[st.cnt * kWave + lane] = pos_base + 8 * q;
        st.cnt += (g[q] >= st.thr) ? 1 : 0;
      }
    }
    // Let the appends complete here: LDS operations share one in-order
    // counter, and with a varying number of them in flight after this branch
    // every later wait for a prefetched operand (the bias) would have to
    // assume the worst case and wait for the appends as well.
    lds_drain();
  }
}

// End of a token block (group log): merge the two logs of each token by
// (logit desc, expert index asc), form the gates and write them to the wave's
// result block `stg` (LDS).  Logits below both halves' thresholds (lower
// bounds of the token's k-th) are skipped.  LSE: pass 1 accumulated the
// full-softmax normaliser and lse goes to the result block (FULL implies it).
// Whole wave active on entry.
template <int KMAX, bool FULL, bool LSE, class PT>
__device__ __forceinline__ void tp_finish_groups(const TwoPassState<KMAX>& st, GroupLog lg, int lane, bool hi_half,
                                                 PT perm, int k, bool want_logit, lds_f32* stg);

// Per-wave result block of the finish: token t (= lane, 0..31) writes entry
// j of its k results at t*k + j of each array, i.e. exactly the order of the
// output rows of the 32 tokens, so the block leaves with a few wide stores.
template <int KMAX>
struct TpStage {
  static constexpr int kIdx = 0, kGate = 32 * KMAX, kLogit = 64 * KMAX, kLse = 96 * KMAX;   // 4-byte words
  static constexpr int kWords = 96 * KMAX + 32;
};

// End of a token block: merge the two logs of each token by (logit desc,
// expert index asc), form the gates and write them to the wave's result
// block `stg` (LDS).  perm: sweep position -> expert (any pointer type).
// Whole wave active on entry.
template <int KMAX, bool FULL, class PT>
__device__ __forceinline__ void tp_finish(const TwoPassState<KMAX>& st, LogRef lg, int lane, bool hi_half, PT perm,
                                          int k, bool want_logit, lds_f32* stg) {
  typedef TpStage<KMAX> S;
  const int cnt_p = (int)partner_u32((uint32_t)st.cnt, hi_half);
  float lse = 0.f;
  if (FULL) {
    // eq. (8) across the two halves of the token
    const float mp = partner_f32(st.m, hi_half), Zp = partner_f32(st.Z, hi_half);
    const float mm = fmaxf(st.m, mp);
    const float Zt = st.Z * __builtin_amdgcn_exp2f((st.m - mm) * kLog2e) +
                     Zp * __builtin_amdgcn_exp2f((mp - mm) * kLog2e);
    lse = mm + __builtin_amdgcn_logf(Zt) * kLn2;
  }
  if (hi_half) return;
  float V[KMAX];
  int IX[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    V[j] = -__builtin_inff();
    IX[j] = 0x7fffffff;
  }
  for (int c = 0; c < st.cnt; ++c) {
    const float2 e = lg.base[c * kWave + lane];
    ordered_insert<KMAX>(V, IX, e.x, perm[__float_as_int(e.y)]);
  }
  int lp = lane + 32;
  asm volatile("" : "+v"(lp));   // recomputed here, not held in a register across the sweeps
  for (int c = 0; c < cnt_p; ++c) {
    const float2 e = lg.base[c * kWave + lp];
    ordered_insert<KMAX>(V, IX, e.x, perm[__float_as_int(e.y)]);
  }
  float w[KMAX];
  if (FULL) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) w[j] = __builtin_amdgcn_exp2f((V[j] - lse) * kLog2e);
  } else {
    // Fig. 12: softmax over the k selected logits, max subtracted
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
  const int o = lane * k;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      stg[S::kIdx + o + j] = __int_as_float(IX[j]);
      stg[S::kGate + o + j] = w[j];
    }
  }
  if (want_logit) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) stg[S::kLogit + o + j] = V[j];
  }
  if (FULL) stg[S::kLse + lane] = lse;
}

// Exact ordering of the logged candidates, branch-free per logit but with
// ~30 VALU per insertion: used only when exact ties decide ranks.
template <int KMAX, class PT>
__device__ __noinline__ void tp_order_groups_slow(GroupLog lg, int lane, int cnt, int cnt_p, float thr, PT perm,
                                                  float* V, int* IX) {
  float v8[KMAX];
  int i8[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    v8[j] = -__builtin_inff();
    i8[j] = 0x7fffffff;
  }
  for (int h = 0; h < 2; ++h) {
    const int ln = lane + 32 * h, n = h ? cnt_p : cnt;
    for (int c = 0; c < n; ++c) {
      const floatx4 v = lg.val[c * kWave + ln];
      const int p = lg.pos[c * kWave + ln];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v[e] >= thr) ordered_insert<KMAX>(v8, i8, v[e], perm[p + e]);
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    V[j] = v8[j];
    IX[j] = i8[j];
  }
}

template <int KMAX, bool FULL, bool LSE, class PT>
__device__ __forceinline__ void tp_finish_groups(const TwoPassState<KMAX>& st, GroupLog lg, int lane, bool hi_half,
                                                 PT perm, int k, bool want_logit, lds_f32* stg) {
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
  // 1. the token's k largest logits: each half's own k largest (med3 lists),
  //    merged across the halves (every logit of the token's top k is logged)
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
  // 2. the selected logits (>= vk) of each half go, with their sweep
  //    positions, straight into the token's result row: the low half fills
  //    it from slot 0 up, the high half from slot k-1 down.  Without exact
  //    ties among them and at the k-th place there are exactly k, so they
  //    fill the row, and the low half then orders the k entries by their rank
  //    in T (the number of larger selected logits).  Otherwise (rare) an
  //    exact merge over both logs rewrites the row.
  const int tok = lane & 31;
  const int o = tok * k;
  const int s0 = hi_half ? o + k - 1 : o;
  const int sd = hi_half ? -1 : 1;
  int nge = 0;
#pragma unroll 2
  for (int c = 0; c < st.cnt; ++c) {
    const floatx4 v = lg.val[c * kWave + lane];
    const int p = lg.pos[c * kWave + lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (v[e] >= vk) {
        if (nge < k) {   // more only with ties: the slots stay in the token's row
          const int sl = s0 + sd * nge;
          stg[S::kLogit + sl] = v[e];
          stg[S::kIdx + sl] = __int_as_float(p + e);
        }
        ++nge;
      }
    }
  }
  bool tie = nge + (int)partner_u32((uint32_t)nge, hi_half) != k;
#pragma unroll
  for (int j = 0; j + 1 < KMAX; ++j) tie = tie || (j >= KMAX - k && T[j] == T[j + 1]);
  float V[KMAX];
  if (!any_lane(tie)) {
    if (hi_half) return;
    float sv[KMAX];
    int sp[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      sv[j] = j < k ? stg[S::kLogit + o + j] : kLowest;
      sp[j] = j < k ? __float_as_int(stg[S::kIdx + o + j]) : 0;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        int r = -(KMAX - k);   // the +inf pads count as larger
#pragma unroll
        for (int i = 0; i < KMAX; ++i) r += T[i] > sv[j] ? 1 : 0;
        stg[S::kIdx + o + r] = __int_as_float((int)perm[sp[j]]);
      }
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) V[j] = T[(j + KMAX - k) < KMAX ? (j + KMAX - k) : KMAX - 1];
  } else {
    if (hi_half) return;
    int IX[KMAX];
    tp_order_groups_slow<KMAX>(lg, lane, st.cnt, cnt_p, thr, perm, V, IX);
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) stg[S::kIdx + o + j] = __int_as_float(IX[j]);
  }
  float w[KMAX];
  if (FULL) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) w[j] = __builtin_amdgcn_exp2f((V[j] - lse) * kLog2e);
  } else {
    // Fig. 12: softmax over the k selected logits, max subtracted
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
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k) stg[S::kGate + o + j] = w[j];
  if (want_logit) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) stg[S::kLogit + o + j] = V[j];
  }
  if (LSE) stg[S::kLse + lane] = lse;
}

}  // namespace more
