// more_split.h -- two-kernel form of the fused low-rank router for gfx950:
// a projection kernel that streams X once and writes z = X R1 (N x r, bf16
// hi + lo, 128 bytes per token at r = 32), then a routing kernel that sweeps
// the experts against z with the exact top-k of more_twopass.h.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.1 Algorithm 1 (phase 1: z = X-block times the
// down-projection; phase 2: one sweep over the experts with a running top-k;
// the N x M logits never reach memory), Fig. 12 and App. F.2.1 eq. (6)/(8)
// for the gates.
//
// Why two kernels on gfx950.  The two phases want different things from a
// compute unit: phase 1 is an HBM stream (all of X, 4 KiB per token at
// h = 2048) that needs ~64 KiB of loads in flight per CU, phase 2 is MFMA +
// VALU work on L2-resident weight tiles that needs those tiles a few hundred
// cycles after asking for them.  Inside one CU the vector-memory path returns
// data in issue order, so when both run side by side every weight tile waits
// behind the X misses queued ahead of it (~2 us), and the sweep stalls; the
// measured time of the one-kernel producer/consumer form is the sum of its
// two halves run alone.  Split, each kernel runs at its own limit, and the
// price is z: 4 % of the X bytes written once and read once.  The logits are
// still formed, filtered and reduced on chip.
//
// Projection kernel: one workgroup per CU holds the packed down-projection
// (A operands of v_mfma_f32_16x16x32_bf16, h*r*2 bytes) in LDS; each
// streaming wave owns 32-token blocks and streams their rows through a ring
// of D register slots (B operand = exactly what a 16-byte load of 16 rows x
// 64 bytes delivers), then leaves z as bf16 hi + lo, in the B-operand layout
// of the 32x32x16 MFMA of the routing kernel, in LDS for a writer wave that
// stores it.
//
// Routing kernel: each wave owns 32-token blocks; it loads z (4 KiB), runs
// the seed pass and the sweep over the expert tiles (weights from L2 through
// a 4-slot register ring, bias and sweep order staged in LDS), merges the
// two half-token logs into its LDS result block and stores that with a few
// 16-byte stores per array.
#pragma once
#include "more_device.h"
#include "more_lowrank.h"
#include "more_pc.h"

namespace more {

// ------------------------------------------------------------- projection
struct ProjArgs {
  const void* X;
  long long N;
  int h;
  const void* R1q;   // [KSQ][R16][64][8] bf16: A operand (R1^T block) of each 32-column K-step
  int KSQ;           // packed K-steps
  int KSP;           // K-steps processed: KSQ rounded up to the ring depth (zero rows in LDS)
  int NB;            // 32-token blocks
  void* Z;           // [NB][hi, lo][R16][64 lanes][16 B]
  int spin_limit;    // polls before a wait gives up
  int* status;       // device word set to a nonzero code if a bounded wait gave up
};

// z bytes of one 32-token block.
__host__ __device__ constexpr int z_block_bytes(int r16) { return 2 * r16 * 1024; }

// LDS map of the projection kernel (bytes): counters | z slots (one per
// streaming wave) | packed down-projection.
constexpr int kPjFlags = 256;   // int full[8], freed[8], abort
template <int R16, int SW>
struct PjLds {
  static constexpr int kSlots = kPjFlags;
  static constexpr int kR1 = kSlots + SW * z_block_bytes(R16);
  static constexpr size_t bytes(int ksp) { return (size_t)kR1 + (size_t)ksp * R16 * 1024; }
};

// SW streaming waves + 1 writer wave.  A streaming wave leaves each block's z
// in its LDS slot and goes on streaming; the writer wave stores it.  Global
// stores share the vector-memory counter with the X loads, which complete in
// issue order: a store in a streaming wave would hold up every X slot issued
// after it until the store is acknowledged, which under the saturated stream
// takes microseconds.  The writer has no loads to wait for.
template <int R16, int D, bool TAIL, int SW>
__global__ __launch_bounds__(64 * (SW + 1)) void proj_kernel(ProjArgs pa) {
  typedef PjLds<R16, SW> L;
  extern __shared__ __align__(16) char pj_lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  {
    // stage the down-projection (K-steps past KSQ are zero): 8 loads in flight
    // per thread, then their stores
    const int n16 = pa.KSP * R16 * 64, q16 = pa.KSQ * R16 * 64;
    const u32x4* src = (const u32x4*)pa.R1q;
    u32x4* dst = (u32x4*)(pj_lds + L::kR1);
    constexpr int T = 64 * (SW + 1), U = 8;
    for (int i0 = 0; i0 < n16; i0 += T * U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * T + (int)threadIdx.x;
        v[u] = i < q16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * T + (int)threadIdx.x;
        if (i < n16) dst[i] = v[u];
      }
    }
    if (threadIdx.x < kPjFlags / 4) ((int*)pj_lds)[threadIdx.x] = 0;
  }
  __syncthreads();
  flag_ptr fl = pc_flags(pj_lds);
  flag_ptr full = fl, freed = fl + 8, abort_word = fl + 16;
  const int W = gridDim.x * SW;   // streaming waves in the grid
  // Work items are 16-token halves of the 32-token blocks (item i: tokens
  // 16i .. 16i + 15, block i / 2), handed out grid-stride: at any time the
  // streaming waves of the grid read adjacent 16-row slabs of X.
  const int NI = 2 * pa.NB;
  auto nitems = [&](int s) { const int w = blockIdx.x * SW + s; return (NI - w + W - 1) / W; };
  auto item = [&](int s, int jj) -> long long { return (long long)(blockIdx.x * SW + s) + (long long)jj * W; };

  if (wave == SW) {
    // writer: serve whichever streaming wave has a block ready
    int served[SW];
#pragma unroll
    for (int s = 0; s < SW; ++s) served[s] = 0;
    for (int idle = 0;;) {
      bool left = false, did = false;
#pragma unroll
      for (int s = 0; s < SW; ++s) {
        if (served[s] >= nitems(s)) continue;
        left = true;
        if (__builtin_amdgcn_readfirstlane(full[s]) <= served[s]) continue;
        asm volatile("" ::: "memory");   // the slot reads stay after the poll
        const char* slot = pj_lds + L::kSlots + s * z_block_bytes(R16);
        u32x4 v[2 * R16];
#pragma unroll
        for (int q = 0; q < 2 * R16; ++q) v[q] = *(const u32x4*)(slot + q * 1024 + lane * 16);
        lds_drain();
        freed[s] = served[s] + 1;
        const long long it = item(s, served[s]);
        const rsrc_t zd = make_rsrc((char*)pa.Z + (size_t)(it >> 1) * z_block_bytes(R16), z_block_bytes(R16));
        // the item's 16 tokens are lanes 16g .. 16g + 15 (mod 32) of the block
        if (((lane >> 4) & 1) == (int)(it & 1)) {
#pragma unroll
          for (int q = 0; q < 2 * R16; ++q) __builtin_amdgcn_raw_buffer_store_b128(v[q], zd, q * 1024 + lane * 16, 0, 0);
        }
        ++served[s];
        did = true;
      }
      if (!left) break;
      if (did) {
        idle = 0;
      } else {
        if (__builtin_amdgcn_readfirstlane(*abort_word) != 0 || ++idle > pa.spin_limit) {
          *abort_word = 1;
          if (pa.status) __hip_atomic_store(pa.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    return;
  }

  const int nj = nitems(wave);
  if (nj <= 0) return;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int rowbytes = pa.h * 2;
  const int vrow0 = l16 * rowbytes;
  const int vx0 = vrow0 + 16 * q4;
  const int NBAT = pa.KSP / D;
  auto xbase = [&](int jj) -> const char* { return (const char*)pa.X + (size_t)item(wave, jj) * 16 * rowbytes; };
  auto xbytes = [&](int jj) -> int {
    if (jj >= nj) return 0;
    const long long rows = pa.N - item(wave, jj) * 16;
    return rows <= 0 ? 0 : (int)((rows < 16 ? rows : 16) * rowbytes);
  };
  lds_cchar* r1l = (lds_cchar*)(pj_lds + L::kR1);
  auto r1op = [&](int s, int rb) -> bf16x8 { return *(lds_cbf16x8*)(r1l + (s * R16 + rb) * 1024 + lane * 16); };
  char* slot = pj_lds + L::kSlots + wave * z_block_bytes(R16);

  // X ring: D slots of one 16-byte load each (the item's 16 rows x 64 bytes
  // of K-step s); each load walks on along the same rows, so the two halves
  // of every 128-byte line are requested back to back.
  bf16x8 xr[D];
  auto issue = [&](int u, rsrc_t xd, int s) {
    if constexpr (TAIL) {
      const int c2 = 64 * s + 16 * q4;   // byte column of this lane's 8 elements
      xr[u] = buf_load(xd, c2 < rowbytes ? vrow0 + c2 : kOob, 0);
    } else {
      xr[u] = buf_load(xd, vx0, 64 * s);
    }
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
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (int jj = 0; jj < nj; ++jj) {
    floatx4 acc[R16];
#pragma unroll
    for (int rb = 0; rb < R16; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[rb][v] = 0.f;
    // down-projection operands: a ring of RP K-steps read from LDS RP-1 steps ahead
    constexpr int RP = 4;
    static_assert(D % RP == 0, "the LDS operand ring must divide the X ring");
    bf16x8 rr[RP][R16];
#pragma unroll
    for (int q = 0; q + 1 < RP; ++q)
#pragma unroll
      for (int rb = 0; rb < R16; ++rb) rr[q][rb] = r1op(q < pa.KSP ? q : pa.KSP - 1, rb);
    for (int sb = 0; sb < NBAT; ++sb) {
      const bool last = sb == NBAT - 1;   // refill with the next item's first K-steps
      const rsrc_t xd = make_rsrc(last ? nbase : cbase, last ? nbytes : cbytes);
      const int s0 = last ? 0 : (sb + 1) * D;
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int s = sb * D + u;
        const int sn = (s + RP - 1 < pa.KSP) ? s + RP - 1 : pa.KSP - 1;
#pragma unroll
        for (int rb = 0; rb < R16; ++rb) rr[(u + RP - 1) % RP][rb] = r1op(sn, rb);
#pragma unroll
        for (int rb = 0; rb < R16; ++rb)
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rr[u % RP][rb], xr[u], acc[rb], 0, 0, 0);
        issue(u, xd, s0 + u);
        // slot order: the MFMAs of slot u wait only for slot u's load
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // acc[rb][v] = z[token 16g + l16][rank 16rb + 4q4 + v] (g = item & 1: the
    // item's half of the block) -> bf16 hi + lo in the 32x32x16 B-operand
    // layout: lane 16g + l16 + 32(q4&1), elements 4(q4>>1) .. +3 of K-step rb;
    // into the slot once the writer has read the previous item out of it
    if (!pc_wait(freed + wave, jj, abort_word, pa.spin_limit)) {
      if (pa.status) __hip_atomic_store(pa.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    {
      const int g = (int)(item(wave, jj) & 1);
      const int off = (16 * g + l16 + 32 * (q4 & 1)) * 16 + 8 * (q4 >> 1);
#pragma unroll
      for (int rb = 0; rb < R16; ++rb) {
        uint32_t hv[2], lv[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float f0 = acc[rb][2 * h2], f1 = acc[rb][2 * h2 + 1];
          const bf16 a0 = (bf16)f0, a1 = (bf16)f1;
          const bf16 b0 = (bf16)(f0 - (float)a0), b1 = (bf16)(f1 - (float)a1);
          hv[h2] = (uint32_t)__builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
          lv[h2] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        }
        *(uint2*)(slot + rb * 1024 + off) = make_uint2(hv[0], hv[1]);
        *(uint2*)(slot + (R16 + rb) * 1024 + off) = make_uint2(lv[0], lv[1]);
      }
    }
    lds_drain();
    full[wave] = jj + 1;
    cbase = nbase;
    cbytes = nbytes;
    nbase = xbase(jj + 2);
    nbytes = xbytes(jj + 2);
  }
}

// ----------------------------------------------------------------- routing
struct RouteArgs {
  LowRankArgs base;   // X unused; NT (multiple of 4), k, R2p, biasp, perm, outputs
  const void* Z;      // as written by proj_kernel
  int NB;             // 32-token blocks
  int pre;            // seed-pass tiles with a bias: a multiple of 4 in [4, NT]
  // non-null: the packed sweep operands come from another stream, which
  // stores `token` (unique to the call) in *ready when they are complete;
  // every workgroup waits for it first (bounded: past spin_limit polls it
  // sets *status and exits)
  const unsigned long long* ready;
  unsigned long long token;
  int spin_limit;
  int* status;
};

template <int KMAX>
struct RouteLds {
  static constexpr int CAPG = KMAX + 2;   // logged 4-logit groups per lane (compacted when full)
  static constexpr int kValBytes = CAPG * kWave * 16;
  static constexpr int kPosBytes = CAPG * kWave * 4;
  static constexpr int kStageBytes = TpStage<KMAX>::kWords * 4;
  static constexpr int kWaveBytes = kValBytes + kPosBytes + kStageBytes;   // per wave: log, result block
  static constexpr size_t bias_off(int waves) { return (size_t)waves * kWaveBytes; }
  static constexpr size_t perm_off(int waves, long long mpad) { return bias_off(waves) + (size_t)mpad * 4; }
  static constexpr size_t flag_off(int waves, long long mpad) { return perm_off(waves, mpad) + (size_t)mpad * 2; }
  static constexpr size_t bytes(int waves, long long mpad) { return flag_off(waves, mpad) + 16; }
};

template <int KMAX, bool FULL, int R16, int WAVES, bool LSE>
__global__ __launch_bounds__(64 * WAVES) void route_kernel(RouteArgs ra) {
  typedef RouteLds<KMAX> L;
  constexpr int CAPG = L::CAPG;
  extern __shared__ __align__(16) char rt_lds[];
  const LowRankArgs& a = ra.base;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NT = a.NT;
  const int mpad = NT * kTile;
  if (ra.ready) {
    lds_i32* word = (lds_i32*)(rt_lds + L::flag_off(WAVES, mpad));
    if (threadIdx.x == 0) {
      // relaxed polls, then one acquire fence (the polls do not invalidate
      // the caches the other workgroups are already filling)
      int ok = 1;
      for (int n = 0; __hip_atomic_load(ra.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != ra.token;) {
        if (++n > ra.spin_limit) {
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      if (!ok && ra.status) __hip_atomic_store(ra.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *word = ok;
    }
    __syncthreads();
    const int ok = *word;
    __syncthreads();   // the word is used again below
    if (!ok) return;   // workgroup-uniform
  }
  // stage the bias (accumulator layout, -inf on padding rows) and the sweep
  // order (position -> expert, 16 bits: M <= 65535 here)
  bool nz = false;   // any nonzero bias
  {
    const float4* src = (const float4*)a.biasp;
    float4* dst = (float4*)(rt_lds + L::bias_off(WAVES));
    for (int i = threadIdx.x; i < mpad / 4; i += 64 * WAVES) {
      const float4 v = src[i];
      dst[i] = v;
      nz = nz || (v.x != 0.f && v.x > -__builtin_inff()) || (v.y != 0.f && v.y > -__builtin_inff()) ||
           (v.z != 0.f && v.z > -__builtin_inff()) || (v.w != 0.f && v.w > -__builtin_inff());
    }
    const int2* psrc = (const int2*)a.perm;
    uint32_t* pdst = (uint32_t*)(rt_lds + L::perm_off(WAVES, mpad));
    for (int i = threadIdx.x; i < mpad / 2; i += 64 * WAVES) {
      const int2 v = psrc[i];
      pdst[i] = ((uint32_t)v.x & 0xffffu) | ((uint32_t)v.y << 16);
    }
  }
  const bool has_bias = block_any(nz, (lds_i32*)(rt_lds + L::flag_off(WAVES, mpad)));
  const int W = gridDim.x * WAVES;
  const int w = blockIdx.x * WAVES + wave;
  const int nj = (ra.NB - w + W - 1) / W;   // blocks of this wave: w, w + W, ...
  if (nj <= 0) return;

  const bool hi = lane >= 32;
  const int hf = hi ? 1 : 0;
  char* wl = rt_lds + wave * L::kWaveBytes;
  const GroupLog lg{(lds_f4*)wl, (lds_i32*)(wl + L::kValBytes)};
  lds_f32* stg = (lds_f32*)(wl + L::kValBytes + L::kPosBytes);
  const float* lb = (const float*)(rt_lds + L::bias_off(WAVES));
  lds_cu16* perm = (lds_cu16*)(rt_lds + L::perm_off(WAVES, mpad));
  const rsrc_t r2d = make_rsrc(a.R2p, NT * R16 * 1024);
  // seed-pass length: without a bias the sweep order carries no hint (plain
  // two passes).  The full-softmax normaliser is accumulated in pass 2, which
  // covers every tile.
  const int P = has_bias ? ra.pre : NT;

  struct Ops {
    bf16x8 w[R16];
  };
  auto load_ops = [&](int t, Ops& o) {
#pragma unroll
    for (int m = 0; m < R16; ++m) o.w[m] = buf_load(r2d, lane * 16 + m * 1024, t * R16 * 1024);
  };
  bf16x8 zh[R16], zl[R16];
  auto load_z = [&](int jj) {
    const rsrc_t zd = make_rsrc((const char*)ra.Z + (size_t)((long long)w + (long long)jj * W) * z_block_bytes(R16),
                                z_block_bytes(R16));
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      zh[m] = buf_load(zd, lane * 16 + m * 1024, 0);
      zl[m] = buf_load(zd, lane * 16 + (R16 + m) * 1024, 0);
    }
  };
  auto bias = [&](int t) -> floatx16 { return *(const floatx16*)(lb + (2 * t + hf) * 16); };
  // logits of one tile, accumulated in place onto its bias
  auto logits = [&](const Ops& o, floatx16& acc) {
#pragma unroll
    for (int m = 0; m < R16; ++m) acc = mfma_bf16(o.w[m], zh[m], acc);
#pragma unroll
    for (int m = 0; m < R16; ++m) acc = mfma_bf16(o.w[m], zl[m], acc);
  };
  auto logits_hi = [&](const Ops& o, floatx16& acc) {
#pragma unroll
    for (int m = 0; m < R16; ++m) acc = mfma_bf16(o.w[m], zh[m], acc);
  };
  // the z-lo products of one tile alternating with the z-hi products of the
  // next: each MFMA depends on the one issued two before it, not on the one
  // just before (the per-tile order of the sums is that of logits())
  auto logits2 = [&](const Ops& o1, floatx16& a1, const Ops& o2, floatx16& a2) {
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      a1 = mfma_bf16(o1.w[m], zl[m], a1);
      a2 = mfma_bf16(o2.w[m], zh[m], a2);
    }
  };

  // Software pipeline over the expert tiles (pass lengths are multiples of
  // 4): tile t lives in slot t % 4 of two 4-slot register rings, its weight
  // operands (o) and its accumulator (ac).  At step t the VALU works on tile
  // t while the MFMAs run that finish tile t+1 (its z-lo products) and start
  // tile t+2 (its z-hi products), alternating, so no MFMA waits for the
  // result of the one issued just before it.  The weight operands of tile
  // t+2 were requested at step t-3 (the newer requests of two steps may
  // still be in flight), and its accumulator was loaded with its bias (LDS)
  // at step t-1, right after tile t-2 left that slot, so the MFMAs
  // accumulate in place.  Every pass starts at tile 0, so near its end both
  // rings are refilled with tiles 0..3 of the next pass (seed pass -> sweep
  // -> next block's seed pass); the last two steps' MFMAs on the next pass's
  // tiles 0 and 1 are discarded and redone when it starts (every step has
  // the same loads and MFMAs, which keeps the wait counts static; the next
  // block's z replaces the current one between the passes).
  Ops o[4];
  floatx16 ac[4];
  load_z(0);
#pragma unroll
  for (int u = 0; u < 4; ++u) load_ops(u, o[u]);
  ac[2] = bias(2);
  // One pass over tiles 0..len-1.  scan(acc, t) is the branch-free work on
  // tile t; it is interleaved with the step's MFMAs (one MFMA, then a few
  // VALU instructions, ...), so the wave keeps issuing while they run.
  // log(acc, t, s) is the rare branchy part.
  auto sweep = [&](int len, auto&& scan, auto&& log) {
    auto wrap = [&](int t) { return t >= len ? t - len : t; };   // t < 2 len
    // the previous pass's last two steps ran their discarded MFMAs on slots 0 and 1
    ac[0] = bias(0);
    ac[1] = bias(1);
    logits(o[0], ac[0]);
    load_ops(wrap(4), o[0]);
    logits_hi(o[1], ac[1]);
    for (int t0 = 0; t0 < len; t0 += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + u;
        const bool last = t == len - 1;   // reload tile 0 of the next pass into its slot
        ac[(u + 3) & 3] = bias(wrap(t + 3));   // the slot of tile t-1, done with at step t-1
        logits2(o[(u + 1) & 3], ac[(u + 1) & 3], o[(u + 2) & 3], ac[(u + 2) & 3]);
        load_ops(last ? 0 : wrap(t + 5), o[(u + 1) & 3]);
        const auto sc = scan(ac[u], t);
#pragma unroll
        for (int m = 0; m < 2 * R16; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // five VALU
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the step order (wait counts rely on it)
        log(ac[u], t, sc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  typedef TpStage<KMAX> S;
  TwoPassState<KMAX> st;
  for (int jj = 0; jj < nj; ++jj) {
    st.init(a.k);
    // pass 1: with a bias, a seed over the first tiles of the bias-descending
    // order bounded by the 4-logit group maxima (closer than the tile maxima,
    // so fewer groups reach the bound in the sweep); without one, a full pass
    // on the tile maxima (group maxima over every tile cost more than they
    // save there)
    sweep(
        P,
        [&](const floatx16& acc, int) {
          if (has_bias)   // workgroup-uniform
            tp_pass1_groups<KMAX>(st, acc);
          else
            tp_pass1_tile<KMAX, false>(st, acc);
          return 0;
        },
        [&](const floatx16&, int, int) {});
    tp_threshold<KMAX>(st, hi, a.k);
    sweep(
        NT,
        [&](const floatx16& acc, int) {
          const floatx4 g = tp_pass2_scan<KMAX, false>(st, acc, false);
          if (LSE) tp_lse_tile<KMAX>(st, acc, g);
          return g;
        },
        [&](const floatx16& acc, int t, const floatx4& g) {
          tp_pass2_groups<KMAX, CAPG>(st, acc, g, kTile * t + 4 * hf, lg, lane, perm, a.k);
        });
    // z of the next block: requested now, behind the ring's refill, so it has
    // arrived by the time the next seed pass starts
    if (jj + 1 < nj) load_z(jj + 1);
    tp_finish_groups<KMAX, FULL, LSE>(st, lg, lane, hi, perm, a.k, a.out_logit != nullptr, stg);
    lds_drain();
    // result block -> memory: one 16-byte store per lane and array (32 k <= 256
    // words); the descriptor range drops the rows past N
    const long long n0 = ((long long)w + (long long)jj * W) * kTile;
    const long long rows = a.N - n0 < kTile ? a.N - n0 : kTile;
    const int bk = (int)rows * a.k * 4;
    lds_cchar* sb = (lds_cchar*)stg;
    const u32x4 vi = lds_ld128(sb, S::kIdx * 4 + lane * 16);
    const u32x4 vg = lds_ld128(sb, S::kGate * 4 + lane * 16);
    __builtin_amdgcn_raw_buffer_store_b128(vi, make_rsrc(a.out_idx + n0 * a.k, bk), lane * 16, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(vg, make_rsrc(a.out_gate + n0 * a.k, bk), lane * 16, 0, 0);
    if (a.out_logit) {
      const u32x4 vl = lds_ld128(sb, S::kLogit * 4 + lane * 16);
      __builtin_amdgcn_raw_buffer_store_b128(vl, make_rsrc(a.out_logit + n0 * a.k, bk), lane * 16, 0, 0);
    }
    if (LSE && a.out_lse) {
      const u32x4 vz = lds_ld128(sb, S::kLse * 4 + lane * 16);
      __builtin_amdgcn_raw_buffer_store_b128(vz, make_rsrc(a.out_lse + n0, (int)rows * 4), lane * 16, 0, 0);
    }
    // the result block is rewritten by the next finish only after these reads
    lds_drain();
  }
}

}  // namespace more
