// more_device.h -- device-side building blocks shared by the MI355X router kernels.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.1 Algorithm 1 (single sweep over the experts with a running
// top-k buffer) and App. F.2.1 eq. (8) (running maximum / normaliser).
//
// CDNA4 mapping used throughout:
//  * Logit tiles come out of a 32x32 MFMA in transposed form: rows are 32
//    experts, columns are 32 tokens.  Lane l (half hf = l/32) owns token l%32
//    and the 16 accumulator rows 8q + 4hf + e (q, e in 0..3), i.e. acc[4q+e].
//    So each token is shared by two lanes, each seeing half of the experts.
//  * Each lane keeps the k best VALUES it has seen as a descending register
//    list updated with v_med3 (k VALU ops per insert, no index bookkeeping),
//    and appends every accepted (value, sweep position) pair to a per-lane
//    log in LDS.  The indices are recovered from the log once at the end.
//  * A candidate must reach the effective threshold max(own k-th, partner's
//    k-th): both are lower bounds of the token's final k-th logit.  Equality
//    is accepted (>=) so that exact ties are resolved at the end by expert
//    index, whatever order the experts were swept in.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace more {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
// Explicit LDS pointers: accesses through them are ds_* instructions (a
// generic pointer may become FLAT, which also waits on the vector-memory counter).
typedef __attribute__((address_space(3))) int lds_i32;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) const uint16_t lds_cu16;
typedef __attribute__((address_space(3))) floatx4 lds_f4;
typedef __attribute__((address_space(3))) const char lds_cchar;
typedef __attribute__((address_space(3))) const u32x4 lds_cu32x4;
typedef __attribute__((address_space(3))) const bf16x8 lds_cbf16x8;
// Wait until every LDS (and scalar-memory) operation of the wave has completed.
// The s_waitcnt builtin (lgkmcnt(0), vmcnt and expcnt at their maxima) is an
// instruction the compiler's own wait-count tracking sees, so it knows the
// counter is empty afterwards; the empty asm keeps memory accesses from
// moving across it.
__device__ __forceinline__ void lds_drain() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
}

// Workgroup-wide OR of v through one LDS word (no static LDS; two barriers).
__device__ __forceinline__ bool block_any(bool v, lds_i32* word) {
  if (threadIdx.x == 0) *word = 0;
  __syncthreads();
  if (v) *word = 1;
  __syncthreads();
  return *word != 0;
}
// 16 bytes of LDS at byte offset off from p (a ds_read_b128)
__device__ __forceinline__ u32x4 lds_ld128(lds_cchar* p, int off) { return *(lds_cu32x4*)(p + off); }

constexpr int kWave = 64;
constexpr int kTile = 32;                // experts per tile == tokens per wave
constexpr float kLowest = -3.4028234663852886e38f;   // -FLT_MAX: start of every list
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ floatx16 mfma_bf16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mfma_f32(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Value held by lane l^32 (the other half of the same token column).
__device__ __forceinline__ uint32_t partner_u32(uint32_t x, bool hi_half) {
  auto pr = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return hi_half ? pr[0] : pr[1];
}
__device__ __forceinline__ float partner_f32(float x, bool hi_half) {
  return __uint_as_float(partner_u32(__float_as_uint(x), hi_half));
}

__device__ __forceinline__ bool any_lane(bool c) {
  return __builtin_amdgcn_ballot_w64(c) != 0;
}

// Log entry: (logit, sweep position) packed in a float2 (position as raw bits).
struct LogRef {
  float2* base;   // this wave's log: entry c of lane l at base[c * 64 + l]
};

// Drop log entries that can no longer reach the top-k (value < thr); returns
// the new entry count.  When exact ties at thr keep the log nearly full, keep
// only the k ties of lowest expert index (the tie rule): entries of higher rank
// among the ties can never be selected.  Called with the whole wave active.
// Kept out of line: it is rare, and its perm[] lookups (global loads) would
// otherwise force conservative memory waits into the sweep loops.  PT: any
// pointer whose [] yields the expert index (global int, or an LDS copy).
template <class PT>
__device__ __noinline__ int compact_log(float2* base, int lane, int cnt, float thr, PT perm, int k, int cap) {
  int w = 0;
  for (int c = 0; c < cnt; ++c) {
    const float2 e = base[c * kWave + lane];
    if (e.x >= thr) {
      base[w * kWave + lane] = e;
      ++w;
    }
  }
  cnt = w;
  if (any_lane(cnt > cap - 8)) {
    if (cnt > cap - 8) {
      // pass 1: knock out ties of rank >= k (rank by original expert index)
      for (int c = 0; c < cnt; ++c) {
        const float2 e = base[c * kWave + lane];
        if (e.x == thr) {
          const int oi = perm[__float_as_int(e.y)];
          int rank = 0;
          for (int c2 = 0; c2 < cnt; ++c2) {
            const float2 e2 = base[c2 * kWave + lane];
            if (e2.x == thr && perm[__float_as_int(e2.y)] < oi) ++rank;
          }
          if (rank >= k) base[c * kWave + lane] = make_float2(-__builtin_inff(), e.y);
        }
      }
      // pass 2: squeeze out the knocked-out entries
      w = 0;
      for (int c = 0; c < cnt; ++c) {
        const float2 e = base[c * kWave + lane];
        if (e.x >= thr) {
          base[w * kWave + lane] = e;
          ++w;
        }
      }
      cnt = w;
    }
  }
  return cnt;
}

template <int KMAX, int CAP>
struct SweepState {
  float L[KMAX];   // descending; the first KMAX-k slots hold +inf (runtime k < KMAX)
  float thr_p;     // partner's k-th (possibly stale: still a valid lower bound)
  float thr;       // max(L[KMAX-1], thr_p)
  int cnt;         // log entries of this lane
  float m, Z;      // running max / normaliser (full-softmax gate only)

  __device__ __forceinline__ void init(int k) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) L[j] = (j < KMAX - k) ? __builtin_inff() : kLowest;
    thr_p = kLowest;
    thr = kLowest;
    cnt = 0;
    m = kLowest * 0.25f;
    Z = 0.f;
  }

  // Insert value x at sweep position pos (lanes masked by the caller).
  __device__ __forceinline__ void insert(float x, int pos, LogRef lg, int lane) {
#pragma unroll
    for (int j = KMAX - 1; j >= 1; --j) L[j] = __builtin_amdgcn_fmed3f(L[j - 1], L[j], x);
    L[0] = fmaxf(L[0], x);
    lg.base[cnt * kWave + lane] = make_float2(x, __int_as_float(pos));
    ++cnt;
    thr = fmaxf(L[KMAX - 1], thr_p);
  }

  __device__ __forceinline__ void compact(LogRef lg, int lane, const int* __restrict__ perm, int k) {
    cnt = compact_log(lg.base, lane, cnt, thr, perm, k, CAP);
  }

  // One 32-expert tile: acc holds this lane's 16 logits (bias included,
  // -inf on padding rows); pos_base = 32*t + 4*hf.
  template <bool FULL>
  __device__ __forceinline__ void tile(const floatx16& acc, int pos_base, LogRef lg, int lane,
                                       bool hi_half, const int* __restrict__ perm, int k) {
    float g[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      g[q] = fmaxf(fmaxf(acc[4 * q], acc[4 * q + 1]), fmaxf(acc[4 * q + 2], acc[4 * q + 3]));
    const float tmax = fmaxf(fmaxf(g[0], g[1]), fmaxf(g[2], g[3]));
    if (FULL) {
      // eq. (8): rescale the running sum when the maximum moves, then add the tile.
      const float mn = fmaxf(m, tmax);
      const float mb = mn * kLog2e;
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) s += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], kLog2e, -mb));
      Z = Z * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + s;
      m = mn;
    }
    thr_p = partner_f32(L[KMAX - 1], hi_half);
    thr = fmaxf(L[KMAX - 1], thr_p);
    if (any_lane(tmax >= thr)) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (any_lane(g[q] >= thr)) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = acc[4 * q + e];
            if (x >= thr) insert(x, pos_base + 8 * q + e, lg, lane);
          }
          if (any_lane(cnt > CAP - 4)) compact(lg, lane, perm, k);
        }
      }
    }
  }
};

// Branch-free variant of SweepState::tile used by the producer/consumer
// kernel: inside a 4-value group that holds a candidate in some lane, every
// value goes through the v_med3 list unconditionally (a value below the list's
// k-th leaves it unchanged, and one between the own k-th and the effective
// threshold only raises the own k-th, which stays a valid lower bound), and is
// written to log slot cnt unconditionally; cnt advances only for values that
// reach the threshold, so rejected writes are overwritten later.  Only the
// tile and group tests branch.
template <int KMAX, int CAP, bool FULL>
__device__ __forceinline__ void tile_bf(SweepState<KMAX, CAP>& st, const floatx16& acc, int pos_base,
                                        LogRef lg, int lane, bool hi_half, const int* __restrict__ perm,
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
          const bool take = x >= st.thr;
          lg.base[st.cnt * kWave + lane] = make_float2(x, __int_as_float(pos_base + 8 * q + e));
          st.cnt += take ? 1 : 0;
#pragma unroll
          for (int j = KMAX - 1; j >= 1; --j) st.L[j] = __builtin_amdgcn_fmed3f(st.L[j - 1], st.L[j], x);
          st.L[0] = fmaxf(st.L[0], x);
          st.thr = fmaxf(st.L[KMAX - 1], st.thr_p);
        }
        if (any_lane(st.cnt > CAP - 4)) st.compact(lg, lane, perm, k);
      }
    }
  }
}

// Tie-aware sorted insertion used once per token at the end: order is
// (value descending, original expert index ascending).
template <int KMAX>
__device__ __forceinline__ void ordered_insert(float (&V)[KMAX], int (&IX)[KMAX], float x, int ix) {
  bool c[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) c[j] = (x > V[j]) || (x == V[j] && ix < IX[j]);
#pragma unroll
  for (int j = KMAX - 1; j >= 1; --j) {
    const float nv = c[j - 1] ? V[j - 1] : (c[j] ? x : V[j]);
    const int ni = c[j - 1] ? IX[j - 1] : (c[j] ? ix : IX[j]);
    V[j] = nv;
    IX[j] = ni;
  }
  if (c[0]) {
    V[0] = x;
    IX[0] = ix;
  }
}

// (v2, i2) ahead of (v, i) in (logit desc, index asc)
__device__ __forceinline__ bool ahead(float v2, int i2, float v, int i) { return v2 > v || (v2 == v && i2 < i); }

// A <- the KMAX best of A and B, both ordered by (logit desc, index asc), in
// that order: A[j] against B[KMAX-1-j] keeps the KMAX best as a bitonic
// sequence, and a bitonic merge network orders it.
template <int KMAX>
__device__ __forceinline__ void bitonic_top(float (&V)[KMAX], int (&IX)[KMAX], const float (&BV)[KMAX],
                                            const int (&BI)[KMAX]) {
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool b = ahead(BV[KMAX - 1 - j], BI[KMAX - 1 - j], V[j], IX[j]);
    V[j] = b ? BV[KMAX - 1 - j] : V[j];
    IX[j] = b ? BI[KMAX - 1 - j] : IX[j];
  }
#pragma unroll
  for (int d = KMAX / 2; d >= 1; d >>= 1) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if ((j & d) == 0) {
        const bool sw = ahead(V[j + d], IX[j + d], V[j], IX[j]);
        const float v = V[j];
        const int x = IX[j];
        V[j] = sw ? V[j + d] : v;
        IX[j] = sw ? IX[j + d] : x;
        V[j + d] = sw ? v : V[j + d];
        IX[j + d] = sw ? x : IX[j + d];
      }
    }
  }
}

// End of a token block: merge the two half-token logs of every token, order
// by (logit desc, expert index asc), form the gates and store.  Must be called
// with the whole wave active (the final compaction uses wave-wide votes).
// SPLIT: each half orders its own log and the halves' lists are merged with a
// bitonic network (for few tokens per wave and long logs, as in the split-M
// form); otherwise the low half orders both logs while the high half waits
// (cheaper when the logs are short).
template <int KMAX, int CAP, bool FULL, bool SPLIT = false>
__device__ __forceinline__ void finish_tokens(SweepState<KMAX, CAP>& st, LogRef lg, int lane,
                                              bool hi_half, bool rowok, long long n,
                                              const int* __restrict__ perm, int k, int* out_idx,
                                              float* out_gate, float* out_logit, float* out_lse) {
  st.thr_p = partner_f32(st.L[KMAX - 1], hi_half);
  st.thr = fmaxf(st.L[KMAX - 1], st.thr_p);
  st.compact(lg, lane, perm, k);
  float lse = 0.f;
  if (FULL) {
    // eq. (8) across the two halves: one running max and one normaliser per token
    const float mp = partner_f32(st.m, hi_half), Zp = partner_f32(st.Z, hi_half);
    const float mm = fmaxf(st.m, mp);
    const float Zt = st.Z * __builtin_amdgcn_exp2f((st.m - mm) * kLog2e) +
                     Zp * __builtin_amdgcn_exp2f((mp - mm) * kLog2e);
    lse = mm + __builtin_amdgcn_logf(Zt) * kLn2;
  }
  float V[KMAX];
  int IX[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    V[j] = -__builtin_inff();
    IX[j] = 0x7fffffff;
  }
  if constexpr (SPLIT) {
    // each half orders its own log, then the two halves' lists are merged
    // (lane l and lane l ^ 32 end with the same KMAX best of the token)
    for (int c = 0; c < st.cnt; ++c) {
      const float2 e = lg.base[c * kWave + lane];
      ordered_insert<KMAX>(V, IX, e.x, perm[__float_as_int(e.y)]);
    }
    float BV[KMAX];
    int BI[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      BV[j] = partner_f32(V[j], hi_half);
      BI[j] = (int)partner_u32((uint32_t)IX[j], hi_half);
    }
    bitonic_top<KMAX>(V, IX, BV, BI);
    if (hi_half || !rowok) return;
  } else {
    const int cnt_p = (int)partner_u32((uint32_t)st.cnt, hi_half);
    if (hi_half || !rowok) return;
    for (int c = 0; c < st.cnt; ++c) {
      const float2 e = lg.base[c * kWave + lane];
      ordered_insert<KMAX>(V, IX, e.x, perm[__float_as_int(e.y)]);
    }
    for (int c = 0; c < cnt_p; ++c) {
      const float2 e = lg.base[c * kWave + lane + 32];
      ordered_insert<KMAX>(V, IX, e.x, perm[__float_as_int(e.y)]);
    }
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
