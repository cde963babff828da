// more_dispatch.h -- kernel selection across the compile units that hold the
// template instances (split so the library builds in parallel).
#pragma once
#include "more_lowrank.h"
#include "more_fullrank.h"
#include "more_stream.h"
#include "more_lock.h"
#include "more_pc.h"
#include "more_split.h"
#include "more_sweep.h"
#include "more_splitm.h"

namespace more {

typedef void (*lowrank_fn)(LowRankArgs);
typedef void (*fullrank_fn)(FullRankArgs);

// Waves per workgroup: each wave's log takes (2*KMAX+8)*512 bytes of LDS;
// keep a workgroup within 64 KiB.
constexpr int waves_for_kmax(int kmax) { return kmax <= 8 ? 4 : (kmax == 16 ? 2 : 1); }

typedef void (*stream_fn)(StreamArgs);

// Ring depth of the streaming kernel: 8 K-steps ahead for r <= 32, 4 for r = 64.
constexpr int stream_depth(int r16) { return r16 <= 2 ? 8 : 4; }
// The streaming kernel covers bf16 storage with r <= 64.
constexpr bool stream_supported(int r16) { return r16 <= 4; }
stream_fn pick_stream(bool full, int kmax, int r16);

// Workgroup-lockstep kernel: bf16, k <= 8, r <= 64, M <= 65536 (16-bit positions).
typedef void (*lock_fn)(LockArgs);
constexpr int kLockKPBM = 4;   // K-steps per batch (max)
constexpr int kLockTPBM = 4;   // expert tiles per batch (max)
constexpr bool lock_supported(int kmax, int r16, long long mpad) {
  return kmax <= 8 && r16 <= 4 && mpad <= 65536;
}
lock_fn pick_lock(bool full, int kmax, int r16, size_t* lds_bytes);

// Producer/consumer kernel: bf16, k <= 8, r <= 64, M <= 65536, LDS within 160 KiB.
typedef void (*pc_fn)(PcArgs);
// Producer ring depth (K-steps in flight): 8 for r <= 32, 4 for r = 64 and for
// the tail instances (h % 32 != 0 or padded K-steps; small odd shapes only).
constexpr int pc_depth(int r16, bool tail) { return (tail || r16 > 2) ? 4 : 8; }
// K-steps of the producer and whether the tail instance is needed.
inline void pc_ksteps(long long h, int r16, int* ksp, bool* tail) {
  const long long ks = (h + 31) / 32;
  *tail = (h % 32 != 0) || (ks % pc_depth(r16, false) != 0);
  const int D = pc_depth(r16, *tail);
  *ksp = (int)((ks + D - 1) / D * D);
}
constexpr long long kLdsBytes = 160 * 1024;
constexpr bool pc_shape_ok(int kmax, int r16, long long mpad) {
  return kmax <= 8 && r16 <= 4 && mpad <= 65536;
}
// Dynamic LDS of the instance for (kmax, r16, mpad); 0 if no instance exists.
size_t pc_lds_bytes(int kmax, int r16, long long mpad);
pc_fn pick_pc(bool full, int kmax, int r16, bool tail);

// Two-kernel form (projection + routing): bf16, k <= 8, r <= 64, M <= 65535.
typedef void (*proj_fn)(ProjArgs);
typedef void (*route_fn)(RouteArgs);
constexpr int kProjWaves = 3;    // projection: three streaming waves + the writer, one per SIMD; one workgroup per CU
constexpr int kRouteWaves = 8;   // routing: eight waves, one workgroup per CU
// Projection ring depth (X loads in flight per wave): 16, or 8 at r = 64,
// where the packed down-projection takes more of the LDS.
constexpr int proj_depth(int r16) { return r16 >= 4 ? 8 : 16; }
// K-steps the projection processes (a multiple of its ring depth) and whether
// the X loads need per-lane column checks.
inline void proj_ksteps(long long h, int r16, int* ksp, bool* tail) {
  const long long ks = (h + 31) / 32;
  const int D = proj_depth(r16);
  *tail = (h % 32 != 0) || (ks % D != 0);
  *ksp = (int)((ks + D - 1) / D * D);
}
constexpr bool split_shape_ok(int kmax, int r16, long long mpad) {
  return kmax <= 8 && r16 <= 4 && mpad <= 65536;   // 16-bit sweep positions
}
proj_fn pick_proj(int r16, bool tail);
// lse: pass 1 over every tile and lse written (the full-softmax gate implies it).
route_fn pick_route(bool full, bool lse, int kmax, int r16);
size_t route_lds_bytes(int kmax, long long mpad);
size_t proj_lds_bytes(int r16, int ksp);
// Expert sweep with the up-projection tiles shared through LDS (the routing
// half of the two-kernel form): bf16, k <= 8, r <= 64, M <= 65536.
typedef void (*sweep_fn)(SweepArgs);
constexpr int kSwCons = 8;   // consumer waves (+ kSwLoaders loaders), one workgroup per CU
sweep_fn pick_sweep(bool full, bool lse, int kmax, int r16);
size_t sweep_lds_bytes(int kmax, int r16);


// Split-M form (few tokens, many experts): bf16, r <= 128, any k.
typedef void (*splitm_proj_fn)(SplitmProjArgs);
typedef void (*splitm_fn)(SplitmArgs);
constexpr int kSplitmMaxBlocks = 64;   // used for at most 64 blocks of 32 tokens
constexpr int kSplitmWaves = 1024;     // routing waves aimed at (blocks x shards)
splitm_proj_fn pick_splitm_proj(int r16);
splitm_fn pick_splitm_topk(int kmax, int r16);
splitm_fn pick_splitm_full(int kmax, int r16);
template <bool FULL, int KMAX>
splitm_fn pick_splitm_r(int r16) {
  switch (r16) {
    case 1: return splitm_route_kernel<KMAX, FULL, 1>;
    case 2: return splitm_route_kernel<KMAX, FULL, 2>;
    case 4: return splitm_route_kernel<KMAX, FULL, 4>;
    default: return splitm_route_kernel<KMAX, FULL, 8>;
  }
}
template <bool FULL>
splitm_fn pick_splitm_k(int kmax, int r16) {
  switch (kmax) {
    case 4: return pick_splitm_r<FULL, 4>(r16);
    case 8: return pick_splitm_r<FULL, 8>(r16);
    case 16: return pick_splitm_r<FULL, 16>(r16);
    default: return pick_splitm_r<FULL, 32>(r16);
  }
}

lowrank_fn pick_lowrank_bf16_topk(int kmax, int r16);
lowrank_fn pick_lowrank_bf16_full(int kmax, int r16);
lowrank_fn pick_lowrank_f32(bool full, int kmax, int r16);
fullrank_fn pick_fullrank(int dt, bool full, int kmax);

template <int DT, int KMAX, bool FULL>
lowrank_fn pick_lowrank_r(int r16) {
  constexpr int W = waves_for_kmax(KMAX);
  switch (r16) {
    case 1: return lowrank_kernel<DT, KMAX, FULL, 1, W>;
    case 2: return lowrank_kernel<DT, KMAX, FULL, 2, W>;
    case 4: return lowrank_kernel<DT, KMAX, FULL, 4, W>;
    default: return lowrank_kernel<DT, KMAX, FULL, 8, W>;
  }
}

template <int DT, bool FULL>
lowrank_fn pick_lowrank_k(int kmax, int r16) {
  switch (kmax) {
    case 4: return pick_lowrank_r<DT, 4, FULL>(r16);
    case 8: return pick_lowrank_r<DT, 8, FULL>(r16);
    case 16: return pick_lowrank_r<DT, 16, FULL>(r16);
    default: return pick_lowrank_r<DT, 32, FULL>(r16);
  }
}

}  // namespace more
