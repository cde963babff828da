// more_pc.h -- producer/consumer form of the fused low-rank router (bf16
// storage, k <= 8, r <= 64, M <= 65536) for gfx950.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.1 Algorithm 1: per block of tokens, phase 1 computes the
// rank-r intermediate z = X-block times the down-projection on chip, phase 2
// sweeps the experts once with a running top-k; only N x k results reach HBM.
//
// The two phases stress different units: phase 1 is a pure HBM stream (all of
// X, ~4 KiB per token at h = 2048) with a little MFMA work, phase 2 is MFMA +
// VALU work on L2-resident weights.  When one wave interleaves both, the HBM
// loads sit in the same in-order vector-memory counter as the short-latency
// weight loads, and either the stream stalls or the sweep waits on HBM.  Here
// the two phases run on different waves of one persistent workgroup per CU:
//
//   4 producer waves (one per SIMD): stream X through a ring of D register
//     slots with v_mfma_f32_16x16x32_bf16, whose B operand is exactly what a
//     16-byte load of 16 rows x 64 bytes delivers (no LDS transpose); at the
//     end of a 32-token block they split z into bf16 hi + lo parts and write
//     them into the LDS slot of the consumer that owns the block;
//   8 consumer waves: read z from their slot (then free it), and compute
//     expert tiles with v_mfma_f32_32x32x16_bf16: logits^T = R2^T z + bias
//     (bias enters as the fp32 accumulator input, staged once in LDS): a
//     short seed pass over the first `pre` tiles of the bias-descending order
//     (pass 1 of more_twopass.h: a lower bound of each token's k-th logit),
//     then one sweep over all tiles that raises the bound and logs what
//     reaches it (tp_sweep_tile).  With a bias, the high-bias tiles at the
//     front hold most of the winners, so the seeded bound is close to the
//     final k-th logit and the log stays short; each expert tile costs ~1.2
//     sweeps instead of 2.
//
// Hand-off: per consumer, two LDS counters (blocks produced / blocks read).
// Each wait is a bounded spin: if a counter does not move within spin_limit
// polls (a protocol error, never expected), the wave sets an abort word that
// every other wave checks at its next wait, so the kernel always terminates.
//
// Block schedule inside workgroup g: local blocks i = 0, 1, ... are global
// blocks g + i*G; producer p streams i = p, p+4, ...; consumer c sweeps
// i = c, c+8, ... (consumers c and c+4 are both fed by producer c%4).
#pragma once
#include "more_device.h"
#include "more_lowrank.h"
#include "more_lock.h"
#include "more_twopass.h"

namespace more {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kPcProd = 4;                     // producer waves per workgroup
constexpr int kPcCons = 8;                     // consumer waves per workgroup
constexpr int kPcWaves = kPcProd + kPcCons;
constexpr int kBufWord3 = 0x00020000;          // raw buffer, 32-bit data format
constexpr int kOob = 0x40000000;               // offset past any descriptor range: loads 0
constexpr int kPcZOff = 256;                   // LDS: hand-off counters, then the z slots
// Seed-pass length in expert tiles (multiple of 4).  With the experts swept in
// bias-descending order, 24 tiles (768 experts) already bound a token's k-th
// logit closely: a simulation of the N(0,1) + N(0,0.5)-bias logits at M = 4096,
// k = 8 logs ~12 entries per token in the sweep (max 24 over 4096 tokens).
constexpr int kPcSeedTiles = 24;

struct PcArgs {
  LowRankArgs base;    // X, N, h, NT (multiple of 4), k, R2p, biasp, perm, outputs
  const void* R1q;     // [KSP][R16][64][8] bf16: A operand (R1^T block) of each K-step
  int NB;              // 32-token blocks
  int G;               // workgroups
  int KSP;             // 32-column K-steps, padded to a multiple of D (zero R1 rows)
  int spin_limit;      // polls before a wait gives up
  int pre;             // seed-pass tiles: a multiple of 4 in [4, NT]
  int* status;         // device word set to a nonzero code if a bounded wait gave up
};

// Hand-off counters (ints at the start of LDS)
constexpr int kPcFull = 0;       // [cons] z blocks published
constexpr int kPcFreed = 8;      // [cons] z blocks read
constexpr int kPcAbort = 16;
constexpr int kPcStaged = 17;    // [cons] result blocks written to the consumer's staging area
constexpr int kPcDrained = 25;   // [cons] result blocks read back out by the producer
constexpr int kPcAnyBias = 63;   // set-up only: does any expert have a nonzero bias

// LDS map (bytes): flags | z slots | logs | result staging | bias | perm (u16)
template <int KMAX, int R16>
struct PcLds {
  static constexpr int CAP = KMAX + 8;     // log entries per lane (compacted when nearly full)
  static constexpr int kZ = kPcZOff;       // [cons][hi, lo][R16][64 lanes][16 B]
  static constexpr int kZBytes = kPcCons * 2 * R16 * 1024;
  static constexpr int kLog = kZ + kZBytes;                            // [cons][CAP][64] (value, position)
  static constexpr int kStage = kLog + kPcCons * CAP * kWave * 8;      // [cons] TpStage<KMAX>
  static constexpr int kStageBytes = TpStage<KMAX>::kWords * 4;
  static constexpr int kBias = kStage + kPcCons * kStageBytes;         // [NT][2][16] f32
  static constexpr size_t perm_off(long long mpad) { return (size_t)kBias + (size_t)mpad * 4; }
  static constexpr size_t bytes(long long mpad) { return perm_off(mpad) + (size_t)mpad * 2; }
};

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufWord3);
}
// AUX = 2: non-temporal (streamed once); 0: default caching.
template <int AUX = 0>
__device__ __forceinline__ bf16x8 buf_load(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}

// The hand-off counters are addressed explicitly in the LDS address space: a
// volatile access through a generic pointer becomes a FLAT instruction, which
// also counts against the vector-memory counter, and waiting for it would
// drain every load in flight (the X ring of a producer, the operand ring of a
// consumer).
typedef volatile lds_i32* flag_ptr;
__device__ __forceinline__ flag_ptr pc_flags(char* lds) { return (flag_ptr)(lds_i32*)lds; }

// Bounded wait until *f >= need.  Returns false (and raises abort) on timeout
// or when another wave has aborted.
__device__ __forceinline__ bool pc_wait(flag_ptr f, int need, flag_ptr abort_word, int limit) {
  for (int it = 0;; ++it) {
    if (__builtin_amdgcn_readfirstlane(*f) >= need) break;
    if (__builtin_amdgcn_readfirstlane(*abort_word) != 0 || it >= limit) {
      *abort_word = 1;
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");   // later LDS reads stay after the poll
  return true;
}

// ------------------------------------------------------------------ producer
// What a producer needs: the token rows, the packed down-projection and the
// block schedule (local block i of workgroup g is global block g + i*G).
struct ProdArgs {
  const void* X;
  long long N;
  int h;
  const void* R1q;   // [KSP][R16][64][8] bf16: A operand (R1^T block) of each K-step
  int KSP;           // 32-column K-steps, padded to a multiple of D (zero R1 rows)
  int G;             // workgroups
};

// Hand-off of the producer/consumer kernel: block i goes to consumer i % 8,
// whose private slot must have been read (freed) first.
//
// The results travel back the same way: a consumer writes each finished
// block into its LDS staging area, and the producer that feeds it (consumer c
// is always fed by producer c % 4) stores them to HBM.  A consumer's global
// stores would otherwise sit in its own vector-memory counter, which counts
// loads and stores in issue order: every later wait for a weight tile would
// also wait for those stores, and under the saturated X stream a store takes
// microseconds to be acknowledged.  In the producer the few stores per block
// are hidden behind the X loads that are in flight anyway.
template <int KMAX, int R16>
struct PcHandOff {
  char* lds;
  int limit;
  int* out_idx;
  float* out_gate;
  float* out_logit;   // may be null
  float* out_lse;     // null unless the full-softmax normaliser is wanted
  long long N;
  int k, G, nbw;

  __device__ __forceinline__ flag_ptr flags() const { return pc_flags(lds); }
  __device__ __forceinline__ char* acquire(int i) const {
    if (!pc_wait(flags() + kPcFreed + i % kPcCons, i / kPcCons, flags() + kPcAbort, limit)) return nullptr;
    return lds + kPcZOff + (i % kPcCons) * 2 * R16 * 1024;
  }
  __device__ __forceinline__ void publish(int i) const {
    lds_drain();
    flags()[kPcFull + i % kPcCons] = i / kPcCons + 1;
  }
  // Store result block r of consumer c (local block c + 8r).
  __device__ __forceinline__ bool drain(int c, int r, int lane) const {
    typedef TpStage<KMAX> S;
    if (!pc_wait(flags() + kPcStaged + c, r + 1, flags() + kPcAbort, limit)) return false;
    const char* stg = lds + PcLds<KMAX, R16>::kStage + c * PcLds<KMAX, R16>::kStageBytes;
    const u32x4 vi = *(const u32x4*)(stg + S::kIdx * 4 + lane * 16);
    const u32x4 vg = *(const u32x4*)(stg + S::kGate * 4 + lane * 16);
    u32x4 vl = {}, vz = {};
    if (out_logit) vl = *(const u32x4*)(stg + S::kLogit * 4 + lane * 16);
    if (out_lse) vz = *(const u32x4*)(stg + S::kLse * 4 + lane * 16);
    lds_drain();
    flags()[kPcDrained + c] = r + 1;
    const long long b = (long long)blockIdx.x + (long long)(c + kPcCons * r) * G;
    const long long n0 = b * kTile;
    const long long rows = N - n0 < kTile ? N - n0 : kTile;
    // one 16-byte store per lane covers a whole array (32 k <= 256 words);
    // the descriptor range drops the lanes past the block's valid rows
    const int bk = (int)rows * k * 4;
    const u32x4 v[2] = {vi, vg};
    void* dst[2] = {out_idx + n0 * k, out_gate + n0 * k};
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_buffer_store_b128(v[q], make_rsrc(dst[q], bk), lane * 16, 0, 0);
    if (out_logit) __builtin_amdgcn_raw_buffer_store_b128(vl, make_rsrc(out_logit + n0 * k, bk), lane * 16, 0, 0);
    if (out_lse) __builtin_amdgcn_raw_buffer_store_b128(vz, make_rsrc(out_lse + n0, (int)rows * 4), lane * 16, 0, 0);
    return true;
  }
  // After block i was handed over: results of consumer i % 8 two rounds back.
  __device__ __forceinline__ bool retire(int i, int lane) const {
    const int r = i / kPcCons - 2;
    return r < 0 || drain(i % kPcCons, r, lane);
  }
  // After the producer's last block: the remaining results of its consumers
  // (the last two rounds of each), older rounds first.
  __device__ __forceinline__ void finish(int p, int lane) const {
    for (int back = 2; back >= 1; --back)
      for (int c = p; c < kPcCons; c += kPcProd) {
        const int r = (nbw - c + kPcCons - 1) / kPcCons - back;   // blocks of consumer c, minus back
        if (r >= 0 && !drain(c, r, lane)) return;
      }
  }
};

// TAIL: h is not a multiple of 32, or the K-steps are padded to a whole ring;
// then the columns past h are replaced by out-of-range offsets (zeros).
// Otherwise every K-step lies inside the row and its column offset is a
// scalar, so the X loads need no per-lane arithmetic at all.
//
// Producer p streams local blocks i = p, p+4, ... and hands each block's z to
// HO as bf16 hi + lo parts in the B-operand layout of the 32x32x16 MFMA
// (HO: acquire(i) -> slot, publish(i), retire(i, lane) after each hand-over,
// finish(p, lane) after the last block).
template <int R16, int D, bool TAIL, class HO>
__device__ __forceinline__ void produce_z(const ProdArgs& pa, const HO& ho, int p, int lane, int nbw) {
  const int nj = (nbw - p + kPcProd - 1) / kPcProd;   // blocks of this producer
  if (nj <= 0) return;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int rowbytes = pa.h * 2;
  const int vrow0 = l16 * rowbytes, vrow1 = (16 + l16) * rowbytes;
  const rsrc_t r1d = make_rsrc(pa.R1q, pa.KSP * R16 * 1024);
  const int NBAT = pa.KSP / D;

  // rows of block jj (fewer at the tail of X; none past the last block)
  auto xbase = [&](int jj) -> const char* {
    const long long b = (long long)blockIdx.x + (long long)(p + kPcProd * jj) * pa.G;
    return (const char*)pa.X + (size_t)b * kTile * rowbytes;
  };
  auto xbytes = [&](int jj) -> int {
    if (jj >= nj) return 0;
    const long long b = (long long)blockIdx.x + (long long)(p + kPcProd * jj) * pa.G;
    const long long rows = pa.N - b * kTile;
    return (int)((rows < kTile ? rows : kTile) * rowbytes);
  };

  bf16x8 xr[D][2], rr[D][R16];
  const int vx0 = vrow0 + 16 * q4, vx1 = vrow1 + 16 * q4;
  auto issue = [&](int u, rsrc_t xd, int s) {
    if constexpr (TAIL) {
      const int c2 = 64 * s + 16 * q4;   // byte column of this lane's 8 elements
      const bool ok = c2 < rowbytes;
      xr[u][0] = buf_load<2>(xd, ok ? vrow0 + c2 : kOob, 0);
      xr[u][1] = buf_load<2>(xd, ok ? vrow1 + c2 : kOob, 0);
    } else {
      xr[u][0] = buf_load<2>(xd, vx0, 64 * s);
      xr[u][1] = buf_load<2>(xd, vx1, 64 * s);
    }
#pragma unroll
    for (int rb = 0; rb < R16; ++rb) rr[u][rb] = buf_load(r1d, lane * 16 + rb * 1024, s * R16 * 1024);
  };

  const char* cbase = xbase(0);
  int cbytes = xbytes(0);
  const char* nbase = xbase(1);
  int nbytes = xbytes(1);
  {
    const rsrc_t xd = make_rsrc(cbase, cbytes);
#pragma unroll
    for (int u = 0; u < D; ++u) {
      issue(u, xd, u);
      __builtin_amdgcn_sched_barrier(0);   // slot order here too (the loop's wait counts assume it)
    }
  }
  for (int jj = 0; jj < nj; ++jj) {
    floatx4 acc[2][R16];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int rb = 0; rb < R16; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[g][rb][v] = 0.f;
    for (int sb = 0; sb < NBAT; ++sb) {
      const bool last = sb == NBAT - 1;   // refill with the next block's first K-steps
      const rsrc_t xd = make_rsrc(last ? nbase : cbase, last ? nbytes : cbytes);
      const int s0 = last ? 0 : (sb + 1) * D;
#pragma unroll
      for (int u = 0; u < D; ++u) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int rb = 0; rb < R16; ++rb)
            acc[g][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rr[u][rb], xr[u][g], acc[g][rb], 0, 0, 0);
        issue(u, xd, s0 + u);
        // keep slot order: the MFMAs of slot u wait only for slot u's loads
        // (D-1 newer slots stay in flight); without the barrier the scheduler
        // groups all MFMAs of a batch ahead of all its loads, which makes every
        // batch wait for the whole ring
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // acc[g][rb][v] = z[token 16g + l16][rank 16rb + 4q4 + v]: hand it over
    const int i = p + kPcProd * jj;
    char* slot = ho.acquire(i);
    if (!slot) return;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      // consumer lane 16g + l16 + 32(q4&1), elements 4(q4>>1) .. +3 of K-step rb
      const int off = (16 * g + l16 + 32 * (q4 & 1)) * 16 + 8 * (q4 >> 1);
#pragma unroll
      for (int rb = 0; rb < R16; ++rb) {
        uint32_t hv[2], lv[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float f0 = acc[g][rb][2 * h2], f1 = acc[g][rb][2 * h2 + 1];
          const bf16 a0 = (bf16)f0, a1 = (bf16)f1;
          const bf16 b0 = (bf16)(f0 - (float)a0), b1 = (bf16)(f1 - (float)a1);
          hv[h2] = (uint32_t)__builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
          lv[h2] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        }
        *(uint2*)(slot + rb * 1024 + off) = make_uint2(hv[0], hv[1]);
        *(uint2*)(slot + (R16 + rb) * 1024 + off) = make_uint2(lv[0], lv[1]);
      }
    }
    ho.publish(i);
    if (!ho.retire(i, lane)) return;
    cbase = nbase;
    cbytes = nbytes;
    nbase = xbase(jj + 2);
    nbytes = xbytes(jj + 2);
  }
  ho.finish(p, lane);
}

// ------------------------------------------------------------------ consumer
template <int KMAX, bool FULL, int R16>
__device__ __forceinline__ void pc_consume(const PcArgs& pa, char* lds, int c, int lane, int nbw, bool has_bias) {
  typedef PcLds<KMAX, R16> L;
  constexpr int CAP = L::CAP;
  const LowRankArgs& a = pa.base;
  const int nj = (nbw - c + kPcCons - 1) / kPcCons;
  if (nj <= 0) return;
  flag_ptr fl = pc_flags(lds);
  flag_ptr abort_word = fl + kPcAbort;
  const bool hi = lane >= 32;
  const int hf = hi ? 1 : 0;
  LogRef lg{(float2*)(lds + L::kLog) + c * CAP * kWave};
  const float* lb = (const float*)(lds + L::kBias);
  const char* slot = lds + L::kZ + c * 2 * R16 * 1024;
  lds_f32* stg = (lds_f32*)(lds + L::kStage + c * L::kStageBytes);
  lds_cu16* perm = (lds_cu16*)(lds + L::perm_off(a.NT * kTile));
  const int NT = a.NT;
  const rsrc_t r2d = make_rsrc(a.R2p, NT * R16 * 1024);

  struct Ops {
    bf16x8 w[R16];
  };
  auto load_ops = [&](int t, Ops& o) {
#pragma unroll
    for (int m = 0; m < R16; ++m) o.w[m] = buf_load(r2d, lane * 16 + m * 1024, t * R16 * 1024);
  };
  bf16x8 zh[R16], zl[R16];
  // bias of tile t in accumulator layout (read one tile ahead of its use)
  auto bias = [&](int t) -> floatx16 { return *(const floatx16*)(lb + (2 * t + hf) * 16); };
  auto logits = [&](const Ops& o, const floatx16& b) -> floatx16 {
    floatx16 acc = b;
#pragma unroll
    for (int m = 0; m < R16; ++m) acc = mfma_bf16(o.w[m], zh[m], acc);
#pragma unroll
    for (int m = 0; m < R16; ++m) acc = mfma_bf16(o.w[m], zl[m], acc);
    return acc;
  };
  // seed-pass length: the full-softmax gate needs pass 1 over every tile, and
  // without a bias the sweep order carries no hint (plain two passes)
  const int P = (FULL || !has_bias) ? NT : pa.pre;

  // Software pipeline over the expert tiles (pass lengths are multiples of 4):
  // at step t the VALU works on tile t while the MFMAs of tile t+1 run; the
  // weight operands of tile t+1 were requested at step t-4 (a 4-slot register
  // ring, so three newer requests may still be in flight: the wait never
  // reaches back to a recent L2 request) and its bias (LDS) at step t-2.
  // Every pass starts at tile 0, so near its end the ring is refilled with
  // tiles 0..3 of the next pass (seed pass -> sweep -> next block's seed).
  Ops o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) load_ops(u, o[u]);
  floatx16 bq[2];
  bq[0] = bias(0);
  bq[1] = bias(1);
  // one pass over tiles 0..len-1; per_tile(acc, t) sees the logits of tile t
  auto sweep = [&](int len, auto&& per_tile) {
    auto wrap = [&](int t) { return t >= len ? t - len : t; };   // t < 2 len
    floatx16 acc[2];
    acc[0] = logits(o[0], bq[0]);
    load_ops(wrap(4), o[0]);
    bq[0] = bias(2);
    for (int t0 = 0; t0 < len; t0 += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + u;
        const bool last = t == len - 1;   // then tile t+1 is the next pass's tile 0 (discarded)
        acc[(u + 1) & 1] = logits(o[(u + 1) & 3], bq[(u + 1) & 1]);
        bq[(u + 1) & 1] = bias(last ? 0 : wrap(t + 3));
        load_ops(last ? 0 : wrap(t + 5), o[(u + 1) & 3]);
        per_tile(acc[u & 1], t);
        __builtin_amdgcn_sched_barrier(0);   // keep the step order (wait counts rely on it)
      }
    }
  };
  TwoPassState<KMAX> st;
  for (int jj = 0; jj < nj; ++jj) {
    if (!pc_wait(fl + kPcFull + c, jj + 1, abort_word, pa.spin_limit)) return;
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      zh[m] = *(const bf16x8*)(slot + m * 1024 + lane * 16);
      zl[m] = *(const bf16x8*)(slot + (R16 + m) * 1024 + lane * 16);
    }
    lds_drain();
    fl[kPcFreed + c] = jj + 1;
    st.init(a.k);
    sweep(P, [&](const floatx16& acc, int) { tp_pass1_tile<KMAX, FULL>(st, acc); });
    tp_threshold<KMAX>(st, hi, a.k);
    sweep(NT, [&](const floatx16& acc, int t) {
      tp_pass2_tile<KMAX, CAP, !FULL>(st, acc, t >= P, kTile * t + 4 * hf, lg, lane, perm, a.k);
    });
    // the staging area must have been read out (block jj-1) before it is rewritten
    if (!pc_wait(fl + kPcDrained + c, jj, abort_word, pa.spin_limit)) return;
    tp_finish<KMAX, FULL>(st, lg, lane, hi, perm, a.k, a.out_logit != nullptr, stg);
    lds_drain();
    fl[kPcStaged + c] = jj + 1;
  }
}

template <int KMAX, bool FULL, int R16, int D, bool TAIL>
__global__ __launch_bounds__(64 * kPcWaves) void pc_kernel(PcArgs pa) {
  typedef PcLds<KMAX, R16> L;
  extern __shared__ __align__(16) char pc_lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // stage the bias (accumulator layout, -inf on padding rows) and the sweep
  // order (position -> expert, 16 bits: M <= 65535 here); clear the counters
  const int mpad = pa.base.NT * kTile;
  const float4* src = (const float4*)pa.base.biasp;
  float4* dst = (float4*)(pc_lds + L::kBias);
  bool nz = false;   // any nonzero bias (padding rows hold -inf)
  for (int i = threadIdx.x; i < mpad / 4; i += 64 * kPcWaves) {
    const float4 v = src[i];
    dst[i] = v;
    nz = nz || (v.x != 0.f && v.x > -__builtin_inff()) || (v.y != 0.f && v.y > -__builtin_inff()) ||
         (v.z != 0.f && v.z > -__builtin_inff()) || (v.w != 0.f && v.w > -__builtin_inff());
  }
  const int2* psrc = (const int2*)pa.base.perm;
  uint32_t* pdst = (uint32_t*)(pc_lds + L::perm_off(mpad));
  for (int i = threadIdx.x; i < mpad / 2; i += 64 * kPcWaves) {
    const int2 v = psrc[i];
    pdst[i] = ((uint32_t)v.x & 0xffffu) | ((uint32_t)v.y << 16);
  }
  if (threadIdx.x < kPcZOff / 4) ((int*)pc_lds)[threadIdx.x] = 0;
  const bool has_bias = block_any(nz, (lds_i32*)pc_lds + kPcAnyBias);
  const int nbw = (pa.NB - (int)blockIdx.x + pa.G - 1) / pa.G;   // blocks of this workgroup
  if (wave < kPcProd)
    produce_z<R16, D, TAIL>(ProdArgs{pa.base.X, pa.base.N, pa.base.h, pa.R1q, pa.KSP, pa.G},
                            PcHandOff<KMAX, R16>{pc_lds, pa.spin_limit, pa.base.out_idx, pa.base.out_gate,
                                                 pa.base.out_logit, FULL ? pa.base.out_lse : nullptr, pa.base.N,
                                                 pa.base.k, pa.G, nbw},
                            wave, lane, nbw);
  else
    pc_consume<KMAX, FULL, R16>(pa, pc_lds, wave - kPcProd, lane, nbw, has_bias);
  // a wave whose bounded wait gave up (or saw another give up) reports it
  asm volatile("" ::: "memory");
  if (pa.status && __builtin_amdgcn_readfirstlane(pc_flags(pc_lds)[kPcAbort]) != 0)
    __hip_atomic_store(pa.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace more
