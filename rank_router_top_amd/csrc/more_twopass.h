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
//     normaliser (eq. 8) is accumulated here too.
//   pass 2: recompute each tile; only lanes with a logit >= thr do anything:
//     they append (logit, sweep position) to their LDS log.  Every logit of
//     the final top-k is >= thr, so it is in one of the token's two logs.
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
template <int KMAX>
__device__ __noinline__ float2 tp_compact(float2* base, int lane, int cnt, float thr,
                                          const int* __restrict__ perm, int k, int cap) {
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
template <int KMAX, int CAP>
__device__ __forceinline__ void tp_pass2_tile(TwoPassState<KMAX>& st, const floatx16& acc, int pos_base,
                                              LogRef lg, int lane, const int* __restrict__ perm, int k) {
  float g[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    g[q] = fmaxf(fmaxf(acc[4 * q], acc[4 * q + 1]), fmaxf(acc[4 * q + 2], acc[4 * q + 3]));
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
  }
}

// End of a token block: merge the two logs of each token by (logit desc,
// expert index asc), form the gates, store.  Whole wave active on entry.
template <int KMAX, bool FULL>
__device__ __forceinline__ void tp_finish(const TwoPassState<KMAX>& st, LogRef lg, int lane, bool hi_half,
                                          bool rowok, long long n, const int* __restrict__ perm, int k,
                                          int* out_idx, float* out_gate, float* out_logit, float* out_lse) {
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
  if (hi_half || !rowok) return;
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
  for (int c = 0; c < cnt_p; ++c) {
    const float2 e = lg.base[c * kWave + lane + 32];
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


}  // namespace more
