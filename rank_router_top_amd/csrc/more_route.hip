// more_route.hip -- host side of libmore_route.so: validation, workspace
// layout and kernel dispatch for the C ABI in include/more_route.h.
//
// Every routing call enqueues two kernels on the caller's stream:
//   1. pack_kernel: the expert sweep order (bias descending) and the weights
//      in MFMA operand order, written into the caller's workspace;
//   2. the fused router kernel (low rank or full rank).
// Nothing is allocated, no state survives the call, no HIP call is made
// before every argument has been checked.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>

#include "more_route.h"
#include "more_device.h"
#include "more_pack.h"
#include "more_order.h"
#include "more_dispatch.h"
#include "more_fullrank_tiled.h"
#include "more_merge.h"
#include "more_balance.h"
#include "more_sort.h"
#include "more_backward.h"

using namespace more;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int kmax_for(int k) { return k <= 4 ? 4 : k <= 8 ? 8 : k <= 16 ? 16 : 32; }
int r16_for(int64_t r) { return r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : 8; }
int waves_for(int kmax) { return waves_for_kmax(kmax); }
size_t log_bytes(int kmax) { return (size_t)(2 * kmax + 8) * kWave * sizeof(float2); }

struct Layout {
  int NT, Mpad, r16, rb, ks1, ks2, ksq, epl, esize;
  size_t off_status, off_r1p, off_r2p, off_bias, off_biasq, off_perm, off_okeys, off_r1q, off_seed, total;
};

// Workspace layout of one call.  All offsets are 256-byte aligned.
bool make_layout(int fullrank, more_dtype dt, int64_t h, int64_t r, int64_t M, Layout* L) {
  L->NT = (int)((M + kTile - 1) / kTile);
  L->NT = (L->NT + 3) / 4 * 4;              // whole groups of 4 tiles (sweep pipelines)
  L->Mpad = L->NT * kTile;
  L->epl = (dt == MORE_DT_BF16) ? 8 : 1;
  L->esize = (dt == MORE_DT_BF16) ? 2 : 4;
  const size_t lane_bytes = (size_t)kWave * L->epl * L->esize;   // one K-step operand
  L->ksq = 0;
  if (fullrank) {
    L->r16 = 0;
    L->rb = 0;
    L->ks1 = 0;
    L->ks2 = (dt == MORE_DT_BF16) ? (int)((h + 15) / 16) : (int)((h + 1) / 2);
  } else {
    L->r16 = r16_for(r);
    L->rb = (L->r16 + 1) / 2;
    L->ks1 = (dt == MORE_DT_BF16) ? (int)((h + 15) / 16) : (int)((h + 1) / 2);
    L->ks2 = (dt == MORE_DT_BF16) ? L->r16 : 8 * L->r16;
    if (dt == MORE_DT_BF16 && stream_supported(L->r16)) {
      // the streaming kernel's ring consumes K-steps in batches of D: pad with
      // zero weight rows so every batch is whole
      const int D = stream_depth(L->r16);
      L->ks1 = (L->ks1 + D - 1) / D * D;
    }
    if (dt == MORE_DT_BF16 && L->r16 <= 4) {
      // producer/consumer kernel: 32-column K-steps in whole batches of its ring depth
      bool tail = false;
      pc_ksteps(h, L->r16, &L->ksq, &tail);
    }
  }
  size_t off = 0;
  // the stall word of the routing kernels' bounded waits (fixed place: offset 0)
  L->off_status = off;
  off += kAlign;
  L->off_r1p = off;
  off += align_up((size_t)L->ks1 * L->rb * lane_bytes);
  L->off_r2p = off;
  off += align_up((size_t)L->NT * L->ks2 * lane_bytes);
  L->off_bias = off;
  off += align_up((size_t)L->NT * 2 * 16 * sizeof(float));
  L->off_biasq = off;
  // rounded up to whole groups of 4 tiles: the lockstep kernel stages bias 1 KiB at a time
  off += align_up((size_t)((L->NT + 3) / 4 * 4) * kWave * sizeof(uint32_t));
  L->off_perm = off;
  off += align_up((size_t)L->Mpad * sizeof(int));
  // sorted chunks of bias keys (the bias-descending order is built from them)
  L->off_okeys = off;
  if (M <= kOrderMaxM)
    off += align_up((size_t)((M + kOrderChunk - 1) / kOrderChunk) * kOrderChunk * sizeof(uint32_t));
  L->off_r1q = off;
  off += align_up((size_t)L->ksq * L->r16 * 1024);
  // weight statistics of the sweep kernel's error bound and seed pass
  // seed-pass length of the LDS-ring sweep
  L->off_seed = off;
  off += kAlign;
  L->total = off;
  return true;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Token scratch after the packed weights: z of every 32-token block for the
// two-kernel path (bf16 storage, r <= 64).  0 where that path cannot run.
size_t z_scratch_bytes(more_dtype dt, const Layout& L, int64_t N) {
  if (dt != MORE_DT_BF16 || L.ksq <= 0 || L.r16 > 4 || N <= 0) return 0;
  const int64_t nb = (N + kTile - 1) / kTile;
  return align_up((size_t)nb * (size_t)z_block_bytes(L.r16));
}

// Split-M form (few tokens, many experts): shards of the sweep tiles and the
// token scratch behind the packed weights.
struct SplitmPlan {
  int NB, S, TPS, KS, KPS;
  size_t off_part, off_cl, off_ci, off_cg, off_lse, bytes;   // offsets from the scratch start
};

bool splitm_plan(more_dtype dt, const Layout& L, int64_t N, int64_t h, int k, SplitmPlan* P) {
  if (dt != MORE_DT_BF16 || N <= 0 || L.r16 > 8) return false;
  const int64_t nb = (N + kTile - 1) / kTile;
  if (nb > kSplitmMaxBlocks) return false;
  // about kSplitmWaves routing waves; shards of a multiple of 4 tiles (so
  // every shard holds a real expert: padding is confined to the last 4 tiles)
  const int64_t want = std::min<int64_t>(std::max<int64_t>(kSplitmWaves / nb, 1), L.NT / 4);
  if (want < 4) return false;
  const int64_t tps = ((L.NT + want - 1) / want + 3) / 4 * 4;
  P->NB = (int)nb;
  P->TPS = (int)tps;
  P->S = (int)((L.NT + tps - 1) / tps);
  P->KS = (int)((h + 15) / 16);
  P->KPS = (P->KS + kSplitmKParts - 1) / kSplitmKParts;
  const int rb = (L.r16 + 1) / 2;
  const size_t cand = align_up((size_t)P->S * (size_t)N * (size_t)k * 4);
  size_t off = 0;
  P->off_part = off;
  off += align_up((size_t)kSplitmKParts * (size_t)nb * rb * 16 * kWave * sizeof(float));
  P->off_cl = off;
  off += cand;
  P->off_ci = off;
  off += cand;
  P->off_cg = off;
  off += cand;
  P->off_lse = off;
  off += align_up((size_t)P->S * (size_t)N * sizeof(float));
  P->bytes = off;
  return true;
}

// Token scratch of a routing call: z for the two-kernel form, or the
// split-M form's partial sums and shard candidates.
size_t token_scratch_bytes(more_dtype dt, const Layout& L, int64_t N, int64_t h, int k) {
  SplitmPlan P;
  const size_t sm = splitm_plan(dt, L, N, h, k, &P) ? P.bytes : 0;
  return std::max(z_scratch_bytes(dt, L, N), sm);
}

// Workspace of the balancing call: packed weights, z scratch for N tokens,
// then the per-slot partial column sums (fp32, by sweep position) and the
// per-slot counts (int32, by expert).  Returns false outside its envelope
// (bf16, r <= 64, k <= 8, the two-kernel path's shape limits).
struct BalLayout {
  size_t off_z, off_part, off_cpart, total;
  int slots;
};
bool balance_layout(more_dtype dt, const Layout& L, int64_t N, int64_t h, int64_t M, int32_t k, BalLayout* B);

more_status validate(int fullrank, more_dtype dt, const void* X, int64_t N, int64_t h,
                     const void* A, int64_t r, const void* B, int64_t M, const float* bias,
                     int32_t k, more_gate gate, const int32_t* idx, const float* gates,
                     const float* logit, const float* lse) {
  if (dt != MORE_DT_BF16 && dt != MORE_DT_F32) return MORE_ERR_BAD_DTYPE;
  if (gate != MORE_GATE_TOPK_SOFTMAX && gate != MORE_GATE_FULL_SOFTMAX) return MORE_ERR_BAD_GATE;
  if (N < 0 || h < 1 || M < 1 || (!fullrank && r < 1)) return MORE_ERR_BAD_SHAPE;
  if (N > (1LL << 40) || h > (1 << 20) || M > (1 << 24) || (!fullrank && r > (1 << 20)))
    return MORE_ERR_BAD_SHAPE;
  if (k < 1 || k > MORE_MAX_K || (int64_t)k > M) return MORE_ERR_BAD_K;
  if (h % 8 != 0) return MORE_ERR_UNSUPPORTED;
  if (!fullrank && (r % 16 != 0 || r > MORE_MAX_R)) return MORE_ERR_UNSUPPORTED;
  if (N == 0) return MORE_OK;
  if (!X || !A || (!fullrank && !B) || !idx || !gates) return MORE_ERR_NULL_ARG;
  if (!aligned16(X) || !aligned16(A) || (!fullrank && !aligned16(B)) || !aligned16(idx) ||
      !aligned16(gates) || (bias && !aligned16(bias)) || (logit && !aligned16(logit)) ||
      (lse && !aligned16(lse)))
    return MORE_ERR_ALIGNMENT;
  return MORE_OK;
}

// ---------------------------------------------------------------- dispatch
// Kernel paths of the low-rank router, in the order they are tried (measured
// fastest first on the workloads they share).  Each call takes the first one
// whose shape envelope fits.  A testing aid can restrict the candidates to a
// subset of "split,ring,splitm,pc,lock,stream" (the plain kernel always remains, so that
// every path can be checked on the shapes a faster one would take): the
// environment variable MORE_ROUTE_PATHS, read once at the first routing call,
// or more_set_route_paths() at any time.
enum { kPathPc = 1, kPathLock = 4, kPathStream = 8, kPathSplit = 16, kPathRing = 32, kPathSplitM = 64, kPathAll = 127 };

int parse_paths(const char* names) {
  if (!names || !*names) return kPathAll;
  int mask = 0;
  static const struct { const char* name; int bit; } table[] = {
      {"split", kPathSplit}, {"ring", kPathRing}, {"splitm", kPathSplitM}, {"pc", kPathPc}, {"lock", kPathLock},
      {"stream", kPathStream}};
  for (const char* p = names; *p;) {
    const char* e = strchr(p, ',');
    const size_t n = e ? (size_t)(e - p) : strlen(p);
    for (const auto& t : table)
      if (n == strlen(t.name) && strncmp(p, t.name, n) == 0) mask |= t.bit;
    if (!e) break;
    p = e + 1;
  }
  return mask;
}

std::atomic<int> g_paths{-1};   // -1: not read from the environment yet
std::atomic<int> g_spin_limit{1 << 22};   // polls before a kernel's bounded wait gives up

bool path_allowed(int path) {
  int m = g_paths.load(std::memory_order_relaxed);
  if (m < 0) {
    int fresh = parse_paths(getenv("MORE_ROUTE_PATHS"));
    g_paths.compare_exchange_strong(m, fresh);
    m = g_paths.load(std::memory_order_relaxed);
  }
  return (m & path) != 0;
}

// Whether the two-kernel path has an instance for this shape (LDS included),
// with the routing kernel reading the R2 tiles itself (ring = false) or
// through the workgroup's LDS ring (ring = true).
bool split_fits(int kmax, const Layout& L, int64_t h, bool ring) {
  if (!split_shape_ok(kmax, L.r16, L.Mpad)) return false;
  int ksp = 0;
  bool tail = false;
  proj_ksteps(h, L.r16, &ksp, &tail);
  const long long rt = ring ? (long long)sweep_lds_bytes(kmax, L.r16) : (long long)route_lds_bytes(kmax, L.Mpad);
  return (long long)proj_lds_bytes(L.r16, ksp) <= kLdsBytes && rt <= kLdsBytes;
}

// Two kernels: projection (R1 resident in LDS) writes z of every 32-token
// block to the token scratch behind the packed weights, routing sweeps it.
// lse_mode: pass 1 covers every tile and lse is written (implied by full).
// Split-M form: projection in K-parts, one wave per (block, shard), then the
// merge of the shards' candidate lists.
more_status launch_splitm(const LowRankArgs& a, const Layout& L, const SplitmPlan& P, int kmax, bool full,
                          char* scratch, hipStream_t stream) {
  SplitmProjArgs pa;
  pa.X = a.X;
  pa.N = a.N;
  pa.h = a.h;
  pa.NB = P.NB;
  pa.KS = P.KS;
  pa.KPS = P.KPS;
  pa.R1p = a.R1p;
  pa.part = (float*)(scratch + P.off_part);
  hipLaunchKernelGGL(pick_splitm_proj(L.r16), dim3((unsigned)(P.NB * kSplitmKParts)), dim3(64), 0, stream, pa);
  if (hipGetLastError() != hipSuccess) return MORE_ERR_HIP;
  SplitmArgs sa;
  sa.base = a;
  sa.part = pa.part;
  sa.NB = P.NB;
  sa.TPS = P.TPS;
  sa.S = P.S;
  sa.cand_logit = (float*)(scratch + P.off_cl);
  sa.cand_idx = (int*)(scratch + P.off_ci);
  sa.cand_gate = (float*)(scratch + P.off_cg);
  sa.shard_lse = full ? (float*)(scratch + P.off_lse) : nullptr;
  splitm_fn rf = full ? pick_splitm_full(kmax, L.r16) : pick_splitm_topk(kmax, L.r16);
  const size_t lds = splitm_lds_bytes(kmax);
  if (hipFuncSetAttribute((const void*)rf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return MORE_ERR_HIP;
  const int rw = P.NB * P.S;
  hipLaunchKernelGGL(rf, dim3((unsigned)((rw + 3) / 4)), dim3(256), lds, stream, sa);
  if (hipGetLastError() != hipSuccess) return MORE_ERR_HIP;
  // the candidates carry global expert indices: shard offset 0
  MergeArgs m;
  m.cand_logit = sa.cand_logit;
  m.cand_idx = sa.cand_idx;
  m.shard_lse = sa.shard_lse;
  m.out_idx = a.out_idx;
  m.out_gate = a.out_gate;
  m.out_logit = a.out_logit;
  m.out_lse = a.out_lse;
  m.N = a.N;
  m.W = 0;
  m.G = P.S;
  m.k = a.k;
  return launch_topk_merge(m, full, stream) == hipSuccess ? MORE_OK : MORE_ERR_HIP;
}

// The side stream's operands-ready word (64 bits): in the stall word's
// 256-byte block, on its own 128-byte line.
constexpr size_t kReadyOffset = 128;

// Side-stream packing (the whole routing call): with join, the packed sweep
// operands come from a side stream that overlapped the projection, and the
// stream waits for join after the projection.  With token instead, the side
// stream stores token in the workspace's ready word when they are complete
// and the routing kernel waits for that word itself, so no cross-stream wait
// stands between the two kernels.
struct SideSync {
  hipEvent_t join = nullptr;
  unsigned long long token = 0;   // 0: none
};

more_status launch_split(const LowRankArgs& a, const Layout& L, int64_t h, int kmax, bool full, bool lse_mode,
                         bool ring, char* ws, hipStream_t stream, SideSync side = SideSync()) {
  int ksp = 0;
  bool tail = false;
  proj_ksteps(h, L.r16, &ksp, &tail);
  const size_t pj_lds = proj_lds_bytes(L.r16, ksp);
  proj_fn pf = pick_proj(L.r16, tail);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipFuncSetAttribute((const void*)pf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)pj_lds) != hipSuccess)
    return MORE_ERR_HIP;
  const int64_t nb = (a.N + kTile - 1) / kTile;
  if (nb > (int64_t)1 << 30) return MORE_ERR_BAD_SHAPE;
  ProjArgs pa;
  pa.X = a.X;
  pa.N = a.N;
  pa.h = (int)h;
  pa.R1q = ws + L.off_r1q;
  pa.KSQ = std::min(L.ksq, ksp);
  pa.KSP = ksp;
  pa.NB = (int)nb;
  pa.Z = ws + L.total;
  pa.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  pa.status = (int*)(ws + L.off_status);
  const int64_t pg = std::max<int64_t>(1, std::min<int64_t>(cus, (2 * nb + kProjWaves - 1) / kProjWaves));
  hipLaunchKernelGGL(pf, dim3((unsigned)pg), dim3(64 * (kProjWaves + 1)), pj_lds, stream, pa);
  if (hipGetLastError() != hipSuccess) return MORE_ERR_HIP;
  if (side.join && (ring || !side.token) && hipStreamWaitEvent(stream, side.join, 0) != hipSuccess)
    return MORE_ERR_HIP;
  if (!ring) {
    // every wave reads the R2 tiles from memory itself
    const size_t rt_lds = route_lds_bytes(kmax, L.Mpad);
    route_fn rf = pick_route(full, lse_mode, kmax, L.r16);
    if (hipFuncSetAttribute((const void*)rf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)rt_lds) != hipSuccess)
      return MORE_ERR_HIP;
    RouteArgs ra;
    ra.base = a;
    ra.ready = side.token ? (const unsigned long long*)(ws + L.off_status + kReadyOffset) : nullptr;
    ra.token = side.token;
    ra.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    ra.status = (int*)(ws + L.off_status);
    ra.base.out_lse = lse_mode ? a.out_lse : nullptr;
    ra.Z = pa.Z;
    ra.NB = (int)nb;
    ra.pre = std::min(L.NT, kPcSeedTiles);
    const int64_t rg = std::max<int64_t>(1, std::min<int64_t>(cus, (nb + kRouteWaves - 1) / kRouteWaves));
    hipLaunchKernelGGL(rf, dim3((unsigned)rg), dim3(64 * kRouteWaves), rt_lds, stream, ra);
    return hipGetLastError() == hipSuccess ? MORE_OK : MORE_ERR_HIP;
  }
  const size_t sw_lds = sweep_lds_bytes(kmax, L.r16);
  sweep_fn sf = pick_sweep(full, lse_mode, kmax, L.r16);
  if (hipFuncSetAttribute((const void*)sf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sw_lds) != hipSuccess)
    return MORE_ERR_HIP;
  SweepArgs sa;
  sa.Z = pa.Z;
  sa.R2p = a.R2p;
  sa.biasq = a.biasq;
  sa.seed = (const int*)(ws + L.off_seed);
  sa.perm = a.perm;
  sa.N = a.N;
  sa.NB = (int)nb;
  sa.NT = L.NT;
  sa.k = a.k;
  sa.out_idx = a.out_idx;
  sa.out_gate = a.out_gate;
  sa.out_logit = a.out_logit;
  sa.out_lse = lse_mode ? a.out_lse : nullptr;
  sa.status = pa.status;
  sa.spin_limit = pa.spin_limit;
  const int64_t sg = std::max<int64_t>(1, std::min<int64_t>(cus, (nb + kSwCons - 1) / kSwCons));
  // the loader's sequence (rounds x (seed + sweep) tiles) must fit an int
  if ((nb / (sg * kSwCons) + 1) * 2 * (int64_t)L.NT >= ((int64_t)1 << 30)) return MORE_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(sf, dim3((unsigned)sg), dim3(64 * (kSwCons + kSwLoaders)), sw_lds, stream, sa);
  return hipGetLastError() == hipSuccess ? MORE_OK : MORE_ERR_HIP;
}

bool balance_layout(more_dtype dt, const Layout& L, int64_t N, int64_t h, int64_t M, int32_t k, BalLayout* B) {
  if (dt != MORE_DT_BF16 || L.ksq <= 0 || L.r16 > 4 || k > 8) return false;
  if (!split_fits(kmax_for(k), L, h, false) && !split_fits(kmax_for(k), L, h, true)) return false;
  const int64_t nb = N > 0 ? (N + kTile - 1) / kTile : 0;
  B->slots = (int)std::min<int64_t>(kBalSlots, std::max<int64_t>(nb, 1));
  B->off_z = L.total;
  B->off_part = B->off_z + z_scratch_bytes(dt, L, N);
  B->off_cpart = B->off_part + align_up((size_t)B->slots * (size_t)L.Mpad * sizeof(float));
  B->total = B->off_cpart + align_up((size_t)B->slots * (size_t)M * sizeof(int));
  return true;
}

lowrank_fn pick_lowrank(more_dtype dt, bool full, int kmax, int r16) {
  if (dt == MORE_DT_BF16) return full ? pick_lowrank_bf16_full(kmax, r16) : pick_lowrank_bf16_topk(kmax, r16);
  return pick_lowrank_f32(full, kmax, r16);
}

}  // namespace

namespace more {
// Stores the call's token in the operands-ready word after the packing
// kernels of a side stream (the kernel boundary has made their writes
// visible at device scope).
__global__ __launch_bounds__(64) void ready_kernel(unsigned long long* ready, unsigned long long token) {
  if (threadIdx.x == 0) __hip_atomic_store(ready, token, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
}  // namespace more

namespace {

// What one launch_pack call enqueues: everything, or the two halves of the
// whole routing call's split (the projection's R1 operands and the stall
// word on the caller's stream; the sweep order, R2, bias and R1 of the other
// kernels on a side stream, overlapping the projection).
enum PackPart { kPackAll, kPackProjection, kPackSweep };

more_status launch_pack(more_dtype dt, int fullrank, const void* A, const void* B, const float* bias,
                        int64_t h, int64_t r, int64_t M, const Layout& L, char* ws,
                        hipStream_t stream, PackPart part = kPackAll) {
  PackArgs p;
  memset(&p, 0, sizeof p);
  p.R1 = fullrank ? nullptr : A;
  p.R2 = fullrank ? A : B;
  p.bias = bias;
  p.h = (int)h;
  p.r = (int)r;
  p.M = (int)M;
  p.Mpad = L.Mpad;
  p.NT = L.NT;
  p.kdim = fullrank ? (int)h : (int)r;
  p.ksteps2 = L.ks2;
  p.ksteps1 = L.ks1;
  p.rb = L.rb;
  p.natural_k = fullrank;
  p.rank_blocks = (L.Mpad + 63) / 64;
  const int r1_total = L.ks1 * L.rb * kWave;
  p.r1_blocks = fullrank ? 0 : (r1_total + 1023) / 1024;
  p.ksq = L.ksq;
  p.r16 = L.r16;
  p.r1q_blocks = (L.ksq * L.r16 * kWave + 1023) / 1024;
  p.R1q = ws + L.off_r1q;
  p.R1p = ws + L.off_r1p;
  p.R2p = ws + L.off_r2p;
  p.biasp = (float*)(ws + L.off_bias);
  p.biasq = (uint32_t*)(ws + L.off_biasq);
  p.perm = (int*)(ws + L.off_perm);
  p.status = (int*)(ws + L.off_status);
  p.seed = (int*)(ws + L.off_seed);
  if (part == kPackProjection) {
    p.rank_blocks = 0;
    p.r1_blocks = 0;
    p.seed = nullptr;
  } else if (part == kPackSweep) {
    p.r1q_blocks = 0;
    p.status = nullptr;
  }
  const bool ordered = bias && M <= kOrderMaxM;
  if (ordered && part != kPackProjection) {
    // sweep order: experts by (bias desc, index asc)
    OrderArgs o;
    o.bias = bias;
    o.M = (int)M;
    o.Mpad = L.Mpad;
    o.keys = (uint32_t*)(ws + L.off_okeys);
    o.perm = p.perm;
    hipLaunchKernelGGL(order_sort_kernel, dim3((unsigned)((M + kOrderChunk - 1) / kOrderChunk)), dim3(kOrderSortThreads),
                       0, stream, o);
    hipLaunchKernelGGL(order_rank_kernel, dim3((unsigned)((L.Mpad + kOrderThreads - 1) / kOrderThreads)),
                       dim3(kOrderThreads), 0, stream, o);
    if (hipGetLastError() != hipSuccess) return MORE_ERR_HIP;
  }
  p.sorted = ordered ? 1 : 0;
  p.seed_tiles = ordered ? std::min(L.NT, kPcSeedTiles) : L.NT;
  const int blocks = std::max(1, p.rank_blocks + p.r1_blocks + p.r1q_blocks);
  if (dt == MORE_DT_BF16)
    hipLaunchKernelGGL(pack_kernel<0>, dim3(blocks), dim3(1024), 0, stream, p);
  else
    hipLaunchKernelGGL(pack_kernel<1>, dim3(blocks), dim3(1024), 0, stream, p);
  return hipGetLastError() == hipSuccess ? MORE_OK : MORE_ERR_HIP;
}

}  // namespace

extern "C" {

int more_abi_version(void) { return MORE_ABI_VERSION; }

void more_set_route_paths(const char* names) { g_paths.store(parse_paths(names), std::memory_order_relaxed); }

void more_set_spin_limit(int polls) {
  g_spin_limit.store(polls > 0 ? polls : (1 << 22), std::memory_order_relaxed);
}

more_status more_route_status(void* workspace, void* stream) {
  if (!workspace) return MORE_ERR_NULL_ARG;
  if (((uintptr_t)workspace % kAlign) != 0) return MORE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  int word = 0;
  if (hipStreamSynchronize(s) != hipSuccess) return MORE_ERR_HIP;
  if (hipMemcpy(&word, workspace, sizeof word, hipMemcpyDeviceToHost) != hipSuccess) return MORE_ERR_HIP;
  if (word == 0) return MORE_OK;
  const int zero = 0;
  if (hipMemcpy(workspace, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess) return MORE_ERR_HIP;
  return MORE_ERR_STALLED;
}

const char* more_status_str(more_status s) {
  switch (s) {
    case MORE_OK: return "ok";
    case MORE_ERR_NULL_ARG: return "required pointer is NULL";
    case MORE_ERR_BAD_SHAPE: return "bad shape (N < 0, h/M/r < 1 or too large)";
    case MORE_ERR_BAD_K: return "bad k (need 1 <= k <= min(M, 32))";
    case MORE_ERR_BAD_DTYPE: return "unknown dtype";
    case MORE_ERR_BAD_GATE: return "unknown gate mode";
    case MORE_ERR_WORKSPACE: return "workspace NULL, too small or not 256-byte aligned";
    case MORE_ERR_UNSUPPORTED: return "unsupported shape (need h % 8 == 0, r % 16 == 0, r <= 128)";
    case MORE_ERR_HIP: return "HIP launch failed";
    case MORE_ERR_ALIGNMENT: return "tensor pointer not 16-byte aligned";
    case MORE_ERR_STALLED: return "a routing kernel's bounded wait gave up (outputs invalid)";
    case MORE_ERR_SCRATCH_LIMIT: return "the call needs more scratch than the library's static buffer holds";
  }
  return "unknown status";
}

size_t more_route_workspace_bytes(int fullrank, more_dtype dt, int64_t N, int64_t h, int64_t r,
                                  int64_t M, int32_t k, more_gate gate, int has_bias) {
  (void)has_bias;
  if (dt != MORE_DT_BF16 && dt != MORE_DT_F32) return 0;
  if (gate != MORE_GATE_TOPK_SOFTMAX && gate != MORE_GATE_FULL_SOFTMAX) return 0;
  if (h < 1 || M < 1 || h % 8 != 0 || k < 1 || k > MORE_MAX_K || (int64_t)k > M) return 0;
  if (!fullrank && (r < 16 || r % 16 != 0 || r > MORE_MAX_R)) return 0;
  if (h > (1 << 20) || M > (1 << 24)) return 0;
  Layout L;
  make_layout(fullrank, dt, h, r, M, &L);
  if (N < 0) return 0;
  if (fullrank && dt == MORE_DT_BF16 && fr_tiled_supported(h, M, k))
    return std::max(L.total, align_up(fr_tiled_bytes(h, M)));
  return L.total + (fullrank ? 0 : token_scratch_bytes(dt, L, N, h, k));
}

more_status more_lowrank_pack(more_dtype dt, const void* R1, int64_t h, int64_t r, const void* R2,
                              int64_t M, const float* bias, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (dt != MORE_DT_BF16 && dt != MORE_DT_F32) return MORE_ERR_BAD_DTYPE;
  if (h < 1 || M < 1 || r < 1 || h > (1 << 20) || M > (1 << 24) || r > (1 << 20)) return MORE_ERR_BAD_SHAPE;
  if (h % 8 != 0 || r % 16 != 0 || r > MORE_MAX_R) return MORE_ERR_UNSUPPORTED;
  if (!R1 || !R2) return MORE_ERR_NULL_ARG;
  if (!aligned16(R1) || !aligned16(R2) || (bias && !aligned16(bias))) return MORE_ERR_ALIGNMENT;
  Layout L;
  make_layout(0, dt, h, r, M, &L);
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace % kAlign) != 0)
    return MORE_ERR_WORKSPACE;
  return launch_pack(dt, 0, R1, R2, bias, h, r, M, L, (char*)workspace, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// The routing call on packed weights.  join: the packed sweep operands are
// still being written on a side stream and this event marks their end; every
// path waits for it before its first kernel that reads them.
more_status route_packed(more_dtype dt, const void* X, int64_t N, int64_t h, int64_t r, int64_t M, int32_t k,
                         more_gate gate, int32_t* topk_idx, float* topk_gate, float* topk_logit, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream, SideSync side = SideSync()) {
  // R1/R2 are not read here; a non-null placeholder keeps the shared validation.
  more_status st = validate(0, dt, X, N, h, X, r, X, M, nullptr, k, gate, topk_idx, topk_gate,
                            topk_logit, lse);
  if (st != MORE_OK || N == 0) return st;
  Layout L;
  make_layout(0, dt, h, r, M, &L);
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace % kAlign) != 0)
    return MORE_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  const bool full = gate == MORE_GATE_FULL_SOFTMAX;
  const int kmax = kmax_for(k);
  const int waves = waves_for(kmax);
  LowRankArgs a;
  a.X = X;
  a.N = N;
  a.h = (int)h;
  a.NT = L.NT;
  a.k = k;
  a.R1p = ws + L.off_r1p;
  a.R2p = ws + L.off_r2p;
  a.biasp = (const float*)(ws + L.off_bias);
  a.biasq = (const uint32_t*)(ws + L.off_biasq);
  a.perm = (const int*)(ws + L.off_perm);
  a.out_idx = topk_idx;
  a.out_gate = topk_gate;
  a.out_logit = topk_logit;
  a.out_lse = full ? lse : nullptr;
  const size_t shmem = (size_t)waves * log_bytes(kmax);
  SplitmPlan sp;
  const size_t zbytes = z_scratch_bytes(dt, L, N);
  const bool splitm = path_allowed(kPathSplitM) && splitm_plan(dt, L, N, h, k, &sp) &&
                      workspace_bytes >= L.total + sp.bytes && splitm_lds_bytes(kmax) <= (size_t)kLdsBytes;
  if (!splitm && zbytes > 0 && workspace_bytes >= L.total + zbytes) {
    if (path_allowed(kPathSplit) && split_fits(kmax, L, h, false))
      return launch_split(a, L, h, kmax, full, full, false, ws, (hipStream_t)stream, side);
    if (path_allowed(kPathRing) && split_fits(kmax, L, h, true))
      return launch_split(a, L, h, kmax, full, full, true, ws, (hipStream_t)stream, side);
  }
  // every other path reads packed sweep operands in its first kernel
  if (side.join && hipStreamWaitEvent((hipStream_t)stream, side.join, 0) != hipSuccess) return MORE_ERR_HIP;
  if (splitm) return launch_splitm(a, L, sp, kmax, full, ws + L.total, (hipStream_t)stream);
  const size_t pc_lds = (dt == MORE_DT_BF16 && L.ksq > 0) ? pc_lds_bytes(kmax, L.r16, L.Mpad) : 0;
  if (pc_lds > 0 && (long long)pc_lds <= kLdsBytes && path_allowed(kPathPc)) {
    // Producer/consumer kernel: one 12-wave workgroup per CU, persistent.
    int ksp = 0;
    bool tail = false;
    pc_ksteps(h, L.r16, &ksp, &tail);
    pc_fn fn = pick_pc(full, kmax, L.r16, tail);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)pc_lds) !=
            hipSuccess)
      return MORE_ERR_HIP;
    PcArgs pa;
    pa.base = a;
    const int64_t nb = (N + kTile - 1) / kTile;
    if (nb > (int64_t)1 << 30) return MORE_ERR_BAD_SHAPE;
    pa.NB = (int)nb;
    pa.G = (int)std::max<int64_t>(1, std::min<int64_t>(cus, nb));
    pa.KSP = L.ksq;
    pa.R1q = ws + L.off_r1q;
    pa.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    pa.status = (int*)(ws + L.off_status);
    pa.pre = std::min(L.NT, kPcSeedTiles);
    hipLaunchKernelGGL(fn, dim3((unsigned)pa.G), dim3(64 * kPcWaves), pc_lds, (hipStream_t)stream, pa);
    return hipGetLastError() == hipSuccess ? MORE_OK : MORE_ERR_HIP;
  }
  if (dt == MORE_DT_BF16 && lock_supported(kmax, L.r16, L.Mpad) && path_allowed(kPathLock)) {
    // Workgroup-lockstep kernel, one 8-wave workgroup per CU, persistent.
    size_t lds = 0;
    lock_fn fn = pick_lock(full, kmax, L.r16, &lds);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
            hipSuccess)
      return MORE_ERR_HIP;
    LockArgs la;
    la.base = a;
    const int64_t nb = (N + kTile - 1) / kTile;
    if (nb > (int64_t)1 << 30) return MORE_ERR_BAD_SHAPE;
    la.NB = (int)nb;
    const int64_t wgs = std::max<int64_t>(1, std::min<int64_t>(cus, (nb + kLockWaves - 1) / kLockWaves));
    la.G = (int)(wgs * kLockWaves);
    la.NI = (int)((nb + la.G - 1) / la.G);
    la.KS = (int)((h + 15) / 16);
    la.NBATCH = std::max((L.NT + kLockTPBM - 1) / kLockTPBM, (la.KS + kLockKPBM - 1) / kLockKPBM);
    hipLaunchKernelGGL(fn, dim3((unsigned)wgs), dim3(64 * kLockWaves), lds, (hipStream_t)stream, la);
    return hipGetLastError() == hipSuccess ? MORE_OK : MORE_ERR_HIP;
  }
  if (dt == MORE_DT_BF16 && stream_supported(L.r16) && path_allowed(kPathStream)) {
    // Persistent grid: as many waves as fit on the device at once, each owning
    // an equal number of 32-token blocks.
    stream_fn fn = pick_stream(full, kmax, L.r16);
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fn, 64 * waves, shmem) !=
            hipSuccess)
      return MORE_ERR_HIP;
    StreamArgs sa;
    sa.base = a;
    const int64_t nb = (N + kTile - 1) / kTile;
    if (nb > (int64_t)1 << 30) return MORE_ERR_BAD_SHAPE;
    sa.NB = (int)nb;
    const int64_t slots = std::max<int64_t>(1, (int64_t)cus * std::max(per_cu, 1) * waves);
    const int64_t per_wave = (nb + slots - 1) / slots;
    sa.G = (int)((nb + per_wave - 1) / per_wave);
    sa.KSP = L.ks1;
    const dim3 grid((unsigned)((sa.G + waves - 1) / waves));
    hipLaunchKernelGGL(fn, grid, dim3(64 * waves), shmem, (hipStream_t)stream, sa);
    return hipGetLastError() == hipSuccess ? MORE_OK : MORE_ERR_HIP;
  }
  const int64_t per_block = (int64_t)waves * kTile;
  const dim3 grid((unsigned)((N + per_block - 1) / per_block));
  hipLaunchKernelGGL(pick_lowrank(dt, full, kmax, L.r16), grid, dim3(64 * waves), shmem,
                     (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? MORE_OK : MORE_ERR_HIP;
}

// Side stream (default priority, no implicit synchronisation with the null
// stream) and fork/join events of the whole routing call, one set per
// device, created on first use.  g_side_mu is held from the fork to the
// caller stream's wait on the join, so the events are never re-recorded by
// another call in between.
constexpr int kSideDevices = 64;
std::mutex g_side_mu;
hipStream_t g_side_stream[kSideDevices] = {};
hipEvent_t g_side_fork[kSideDevices] = {};
hipEvent_t g_side_join[kSideDevices] = {};

// Tokens of the ready word: unique per call in this process, counted from a
// clock-derived base, so a stale word (an earlier call's token, or whatever
// the caller's memory held) does not hold the current one.
unsigned long long next_token() {
  static std::atomic<unsigned long long> next{
      ((unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() * 0x9E3779B97F4A7C15ull) | 1ull};
  const unsigned long long t = next.fetch_add(1, std::memory_order_relaxed);
  return t ? t : next.fetch_add(1, std::memory_order_relaxed);
}

bool side_stream(int dev) {
  if (dev < 0 || dev >= kSideDevices) return false;
  if (g_side_stream[dev]) return true;
  hipStream_t s = nullptr;
  hipEvent_t f = nullptr, j = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return false;
  if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
    if (f) (void)hipEventDestroy(f);
    (void)hipStreamDestroy(s);
    return false;
  }
  g_side_stream[dev] = s;
  g_side_fork[dev] = f;
  g_side_join[dev] = j;
  return true;
}

}  // namespace

extern "C" {

more_status more_lowrank_route_packed(more_dtype dt, const void* X, int64_t N, int64_t h, int64_t r,
                                      int64_t M, int32_t k, more_gate gate, int32_t* topk_idx,
                                      float* topk_gate, float* topk_logit, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return route_packed(dt, X, N, h, r, M, k, gate, topk_idx, topk_gate, topk_logit, lse, workspace,
                      workspace_bytes, stream);
}

more_status more_route_lowrank(more_dtype dt, const void* X, int64_t N, int64_t h, const void* R1,
                               int64_t r, const void* R2, int64_t M, const float* bias, int32_t k,
                               more_gate gate, int32_t* topk_idx, float* topk_gate,
                               float* topk_logit, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  more_status st = validate(0, dt, X, N, h, R1, r, R2, M, bias, k, gate, topk_idx, topk_gate,
                            topk_logit, lse);
  if (st != MORE_OK || N == 0) return st;
  Layout L;
  make_layout(0, dt, h, r, M, &L);
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace % kAlign) != 0)
    return MORE_ERR_WORKSPACE;
  const hipStream_t hs = (hipStream_t)stream;
  char* ws = (char*)workspace;
  int dev = -1;
  // bf16 with a bias: the sweep order and the sweep operands are packed on a
  // side stream while the projection (which needs only its own R1 operands)
  // runs on the caller's stream
  if (dt == MORE_DT_BF16 && bias && M <= kOrderMaxM && L.ksq > 0 && hipGetDevice(&dev) == hipSuccess) {
    std::lock_guard<std::mutex> guard(g_side_mu);
    if (side_stream(dev)) {
      const hipStream_t side = g_side_stream[dev];
      // Under graph capture the call's token would be replayed unchanged, so
      // there the caller's stream waits for the side stream's event instead.
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(hs, &cap) != hipSuccess) return MORE_ERR_HIP;
      SideSync sync;
      sync.join = g_side_join[dev];
      if (cap == hipStreamCaptureStatusNone) sync.token = next_token();
      if (hipEventRecord(g_side_fork[dev], hs) != hipSuccess ||
          hipStreamWaitEvent(side, g_side_fork[dev], 0) != hipSuccess)
        return MORE_ERR_HIP;
      st = launch_pack(dt, 0, R1, R2, bias, h, r, M, L, ws, side, kPackSweep);
      if (st == MORE_OK && sync.token) {
        hipLaunchKernelGGL(ready_kernel, dim3(1), dim3(64), 0, side,
                           (unsigned long long*)(ws + L.off_status + kReadyOffset), sync.token);
        if (hipGetLastError() != hipSuccess) st = MORE_ERR_HIP;
      }
      if (hipEventRecord(g_side_join[dev], side) != hipSuccess) return MORE_ERR_HIP;
      if (st == MORE_OK) st = launch_pack(dt, 0, R1, R2, bias, h, r, M, L, ws, hs, kPackProjection);
      if (st == MORE_OK)
        st = route_packed(dt, X, N, h, r, M, k, gate, topk_idx, topk_gate, topk_logit, lse, workspace,
                          workspace_bytes, stream, sync);
      // With a token the routing kernel waited for the side stream's results,
      // so the caller's stream needs no wait; under capture and on an error it
      // still joins the side stream (a capture must rejoin every stream it
      // forked).
      if (st != MORE_OK || !sync.token) (void)hipStreamWaitEvent(hs, g_side_join[dev], 0);
      return st;
    }
  }
  st = launch_pack(dt, 0, R1, R2, bias, h, r, M, L, ws, hs);
  if (st != MORE_OK) return st;
  return route_packed(dt, X, N, h, r, M, k, gate, topk_idx, topk_gate, topk_logit, lse, workspace,
                      workspace_bytes, stream);
}

size_t more_balance_workspace_bytes(more_dtype dt, int64_t N, int64_t h, int64_t r, int64_t M, int32_t k) {
  if (more_route_workspace_bytes(0, dt, N, h, r, M, k, MORE_GATE_TOPK_SOFTMAX, 0) == 0) return 0;
  Layout L;
  make_layout(0, dt, h, r, M, &L);
  BalLayout B;
  return balance_layout(dt, L, N, h, M, k, &B) ? B.total : 0;
}

more_status more_lowrank_balance_packed(more_dtype dt, const void* X, int64_t N, int64_t h, int64_t r,
                                        int64_t M, int32_t k, more_gate gate, int32_t* topk_idx,
                                        float* topk_gate, float* topk_logit, float* lse, float* psum,
                                        int32_t* counts, float* stats, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  more_status st = validate(0, dt, X, N, h, X, r, X, M, nullptr, k, gate, topk_idx, topk_gate,
                            topk_logit, lse);
  if (st != MORE_OK || N == 0) return st;
  if (!lse || !psum || !counts || !stats) return MORE_ERR_NULL_ARG;
  if (!aligned16(psum) || !aligned16(counts) || !aligned16(stats)) return MORE_ERR_ALIGNMENT;
  Layout L;
  make_layout(0, dt, h, r, M, &L);
  BalLayout B;
  if (!balance_layout(dt, L, N, h, M, k, &B)) return MORE_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < B.total || ((uintptr_t)workspace % kAlign) != 0)
    return MORE_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  hipStream_t hs = (hipStream_t)stream;
  const bool full = gate == MORE_GATE_FULL_SOFTMAX;
  LowRankArgs a;
  memset(&a, 0, sizeof a);
  a.X = X;
  a.N = N;
  a.h = (int)h;
  a.NT = L.NT;
  a.k = k;
  a.R1p = ws + L.off_r1p;
  a.R2p = ws + L.off_r2p;
  a.biasp = (const float*)(ws + L.off_bias);
  a.biasq = (const uint32_t*)(ws + L.off_biasq);
  a.perm = (const int*)(ws + L.off_perm);
  a.out_idx = topk_idx;
  a.out_gate = topk_gate;
  a.out_logit = topk_logit;
  a.out_lse = lse;
  // 1. forward: z to the scratch, top-k + gates + lse (pass 1 over every tile)
  st = launch_split(a, L, h, kmax_for(k), full, true, !split_fits(kmax_for(k), L, h, false), ws, hs);
  if (st != MORE_OK) return st;
  // 2. second sweep: psum; counts; column sums; L_bal and H_norm
  const int64_t nb = (N + kTile - 1) / kTile;
  PsumArgs pa;
  pa.Z = ws + B.off_z;
  pa.lse = lse;
  pa.R2p = a.R2p;
  pa.biasp = a.biasp;
  pa.part = (float*)(ws + B.off_part);
  pa.N = N;
  pa.NB = (int)nb;
  pa.NT = L.NT;
  pa.G = (L.NT + kBalWaves * bal_tiles(L.r16) - 1) / (kBalWaves * bal_tiles(L.r16));
  pa.slots = B.slots;
  CountArgs ca;
  ca.idx = topk_idx;
  ca.cpart = (int*)(ws + B.off_cpart);
  ca.N = N;
  ca.k = k;
  ca.M = (int)M;
  ca.NB = (int)nb;
  ca.slots = B.slots;
  ColsumArgs sa;
  sa.part = pa.part;
  sa.cpart = ca.cpart;
  sa.perm = a.perm;
  sa.psum = psum;
  sa.counts = counts;
  sa.M = (int)M;
  sa.Mpad = L.Mpad;
  sa.slots = B.slots;
  StatsArgs ta;
  ta.psum = psum;
  ta.counts = counts;
  ta.stats = stats;
  ta.N = N;
  ta.k = k;
  ta.M = (int)M;
  return launch_balance(L.r16, pa, ca, sa, ta, hs) == hipSuccess ? MORE_OK : MORE_ERR_HIP;
}

namespace {
// Workspace of the backward call: packed weights, z scratch for N tokens,
// then the backward's own area.
struct BwdLayout {
  size_t off_z, off_pbq, off_pbpos, off_r2b, off_r2t, off_inv, off_sel, off_g, off_zbar, off_zrm, off_r2part,
      off_bpart, off_r1part, total;
  int slotsE, slotsX, GE, GX;
};
bool backward_layout(more_dtype dt, const Layout& L, int64_t N, int64_t h, int64_t r, int64_t M, int32_t k,
                     BwdLayout* B) {
  if (dt != MORE_DT_BF16 || L.ksq <= 0 || L.r16 > 2 || r % 16 != 0 || h % kTile != 0 || k > 32) return false;
  if (L.Mpad > 16384) return false;   // bias + pbar of every tile stay in the token kernel's LDS
  int ksp = 0;
  bool tail = false;
  proj_ksteps(h, L.r16, &ksp, &tail);
  if ((long long)proj_lds_bytes(L.r16, ksp) > kLdsBytes) return false;
  const int64_t nb = N > 0 ? (N + kTile - 1) / kTile : 0;
  B->slotsE = (int)std::min<int64_t>(kBwdSlots, std::max<int64_t>(nb, 1));
  B->slotsX = B->slotsE;
  B->GE = (L.NT + kBwdExpWaves * kBwdExpTiles - 1) / (kBwdExpWaves * kBwdExpTiles);
  B->GX = (int)((h / kTile + kBwdXWaves * kBwdXTiles - 1) / (kBwdXWaves * kBwdXTiles));
  const size_t nrow = (size_t)std::max<int64_t>(nb, 1) * kTile;
  size_t off = L.total;
  B->off_z = off;
  off += z_scratch_bytes(dt, L, N);
  B->off_pbq = off;
  off += align_up((size_t)L.NT * 32 * sizeof(float));
  B->off_pbpos = off;
  off += align_up((size_t)L.Mpad * sizeof(float));
  B->off_r2b = off;
  off += align_up((size_t)L.NT * 2048);
  B->off_r2t = off;
  off += align_up((size_t)M * kBwdRow * 2);
  B->off_inv = off;
  off += align_up((size_t)M * sizeof(int));
  B->off_sel = off;
  off += align_up((size_t)std::max<int64_t>(N, 1) * (size_t)k * sizeof(int));
  B->off_g = off;
  off += align_up(nrow * sizeof(float));
  B->off_zbar = off;
  off += align_up(nrow * kBwdRow * sizeof(float));
  B->off_zrm = off;
  off += align_up(nrow * kBwdRow * sizeof(float));
  B->off_r2part = off;
  off += align_up((size_t)B->slotsE * kBwdRow * L.Mpad * sizeof(float));
  B->off_bpart = off;
  off += align_up((size_t)B->slotsE * L.Mpad * sizeof(float));
  B->off_r1part = off;
  off += align_up((size_t)B->slotsX * (size_t)h * kBwdRow * sizeof(float));
  B->total = off;
  return true;
}
}  // namespace

size_t more_backward_workspace_bytes(more_dtype dt, int64_t N, int64_t h, int64_t r, int64_t M, int32_t k) {
  if (more_route_workspace_bytes(0, dt, N, h, r, M, k, MORE_GATE_TOPK_SOFTMAX, 0) == 0) return 0;
  Layout L;
  make_layout(0, dt, h, r, M, &L);
  BwdLayout B;
  return backward_layout(dt, L, N, h, r, M, k, &B) ? B.total : 0;
}

more_status more_lowrank_backward_packed(more_dtype dt, const void* X, int64_t N, int64_t h, const void* R1,
                                         int64_t r, const void* R2, int64_t M, int32_t k, const int32_t* topk_idx,
                                         const float* topk_logit_grad, const float* psum_grad, const float* lse,
                                         void* X_grad, float* R1_grad, float* R2_grad, float* bias_grad,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  more_status st = validate(0, dt, X, N, h, R1, r, R2, M, nullptr, k, MORE_GATE_TOPK_SOFTMAX, topk_idx,
                            topk_logit_grad, nullptr, lse);
  if (st != MORE_OK || N == 0) return st;
  if (!lse || !X_grad || !R1_grad || !R2_grad) return MORE_ERR_NULL_ARG;
  if (!aligned16(X_grad) || !aligned16(R1_grad) || !aligned16(R2_grad) || (psum_grad && !aligned16(psum_grad)) ||
      (bias_grad && !aligned16(bias_grad)))
    return MORE_ERR_ALIGNMENT;
  Layout L;
  make_layout(0, dt, h, r, M, &L);
  BwdLayout B;
  if (!backward_layout(dt, L, N, h, r, M, k, &B)) return MORE_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < B.total || ((uintptr_t)workspace % kAlign) != 0) return MORE_ERR_WORKSPACE;
  const int64_t nb = (N + kTile - 1) / kTile;
  if (nb > (int64_t)1 << 30) return MORE_ERR_BAD_SHAPE;
  char* ws = (char*)workspace;
  hipStream_t hs = (hipStream_t)stream;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MORE_ERR_HIP;
  // 1. recompute z (Algorithm 3, phase 1) into the token scratch
  int ksp = 0;
  bool tail = false;
  proj_ksteps(h, L.r16, &ksp, &tail);
  const size_t pj_lds = proj_lds_bytes(L.r16, ksp);
  proj_fn pf = pick_proj(L.r16, tail);
  if (hipFuncSetAttribute((const void*)pf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)pj_lds) != hipSuccess)
    return MORE_ERR_HIP;
  ProjArgs pa;
  pa.X = X;
  pa.N = N;
  pa.h = (int)h;
  pa.R1q = ws + L.off_r1q;
  pa.KSQ = std::min(L.ksq, ksp);
  pa.KSP = ksp;
  pa.NB = (int)nb;
  pa.Z = ws + B.off_z;
  pa.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  pa.status = (int*)(ws + L.off_status);
  const int64_t pg = std::max<int64_t>(1, std::min<int64_t>(cus, (2 * nb + kProjWaves - 1) / kProjWaves));
  hipLaunchKernelGGL(pf, dim3((unsigned)pg), dim3(64 * (kProjWaves + 1)), pj_lds, hs, pa);
  if (hipGetLastError() != hipSuccess) return MORE_ERR_HIP;
  // 2. phase 2 (two sweeps) and phase 3
  BwdArgs a;
  memset(&a, 0, sizeof a);
  a.Z = ws + B.off_z;
  a.lse = lse;
  a.R2p = ws + L.off_r2p;
  a.biasp = (const float*)(ws + L.off_bias);
  a.perm = (const int*)(ws + L.off_perm);
  a.X = (const uint16_t*)X;
  a.R1 = (const uint16_t*)R1;
  a.R2 = (const uint16_t*)R2;
  a.idx = topk_idx;
  a.tv = topk_logit_grad;
  a.pbar = psum_grad;
  a.pbq = (float*)(ws + B.off_pbq);
  a.pbpos = (float*)(ws + B.off_pbpos);
  a.R2b = (uint16_t*)(ws + B.off_r2b);
  a.R2t = (uint16_t*)(ws + B.off_r2t);
  a.invpos = (int*)(ws + B.off_inv);
  a.selpos = (int*)(ws + B.off_sel);
  a.g = (float*)(ws + B.off_g);
  a.zbar = (float*)(ws + B.off_zbar);
  a.zrm = (float*)(ws + B.off_zrm);
  a.r2part = (float*)(ws + B.off_r2part);
  a.bpart = (float*)(ws + B.off_bpart);
  a.r1part = (float*)(ws + B.off_r1part);
  a.xbar = (uint16_t*)X_grad;
  a.r1grad = R1_grad;
  a.r2grad = R2_grad;
  a.bgrad = bias_grad;
  a.N = N;
  a.h = (int)h;
  a.r = (int)r;
  a.M = (int)M;
  a.k = k;
  a.NT = L.NT;
  a.NB = (int)nb;
  a.slotsE = B.slotsE;
  a.GE = B.GE;
  a.slotsX = B.slotsX;
  a.GX = B.GX;
  const size_t tok_lds = (size_t)L.NT * 32 * sizeof(float) * 2;
  return launch_backward(L.r16, a, tok_lds, cus, hs) == hipSuccess ? MORE_OK : MORE_ERR_HIP;
}

size_t more_dispatch_workspace_bytes(int64_t N, int32_t k, int64_t M) {
  if (N < 0 || k < 1 || M < 1 || M > (1 << 24) || (int64_t)k > M || N * (int64_t)k >= ((int64_t)1 << 31) - 1)
    return 0;
  const int64_t n = N * k;
  size_t bytes = align_up(sort_hist_ints(n, M) * sizeof(int));
  if (sort_passes(M) > 1) bytes += 2 * align_up((size_t)(n > 0 ? n : 1) * sizeof(int));
  return bytes;
}

}  // extern "C"

// Scratch of more_dispatch_sort_noalloc: a file-scope device array (one copy
// on every GPU the library runs on, held until the process ends).  Host code
// must not pass its name to a kernel (on the host it is a stand-in, not a
// device address): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept in g_noalloc_ptr.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

// Argument checks shared by both dispatch-sort entry points (no HIP call).
more_status dispatch_sort_check(const int32_t* topk_idx, int64_t N, int32_t k, int64_t M, const int32_t* sorted_expert,
                                const int32_t* sorted_slot, const int32_t* offsets) {
  if (N < 0 || M < 1 || M > (1 << 24)) return MORE_ERR_BAD_SHAPE;
  if (k < 1 || (int64_t)k > M) return MORE_ERR_BAD_K;
  if (N * (int64_t)k >= ((int64_t)1 << 31) - 1) return MORE_ERR_BAD_SHAPE;
  if (N == 0) return MORE_OK;
  if (!topk_idx || !sorted_expert || !sorted_slot || !offsets) return MORE_ERR_NULL_ARG;
  if (!aligned16(topk_idx) || !aligned16(sorted_expert) || !aligned16(sorted_slot) || !aligned16(offsets))
    return MORE_ERR_ALIGNMENT;
  return MORE_OK;
}

// The sort itself on a checked call; ws holds more_dispatch_workspace_bytes(N, k, M) bytes.
more_status dispatch_sort_run(const int32_t* topk_idx, int64_t N, int32_t k, int64_t M, int32_t* sorted_expert,
                              int32_t* sorted_slot, int32_t* offsets, char* ws, hipStream_t stream) {
  const int n = (int)(N * k);
  int* hist = (int*)ws;
  int* tk = nullptr;
  int* tv = nullptr;
  if (sort_passes(M) > 1) {
    const size_t off = align_up(sort_hist_ints(n, M) * sizeof(int));
    tk = (int*)(ws + off);
    tv = (int*)(ws + off + align_up((size_t)n * sizeof(int)));
  }
  return launch_dispatch_sort(topk_idx, n, (int)M, sorted_expert, sorted_slot, offsets, hist, tk, tv, stream) ==
                 hipSuccess
             ? MORE_OK
             : MORE_ERR_HIP;
}

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};

// Device address of the current device's scratch copy, or nullptr on a HIP error.
void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> guard(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_noalloc_ptr[dev] = p;
  }
  return g_noalloc_ptr[dev];
}

}  // namespace

extern "C" {

more_status more_dispatch_sort(const int32_t* topk_idx, int64_t N, int32_t k, int64_t M, int32_t* sorted_expert,
                               int32_t* sorted_slot, int32_t* offsets, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const more_status c = dispatch_sort_check(topk_idx, N, k, M, sorted_expert, sorted_slot, offsets);
  if (c != MORE_OK || N == 0) return c;
  const size_t need = more_dispatch_workspace_bytes(N, k, M);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign) != 0) return MORE_ERR_WORKSPACE;
  return dispatch_sort_run(topk_idx, N, k, M, sorted_expert, sorted_slot, offsets, (char*)workspace,
                           (hipStream_t)stream);
}

more_status more_dispatch_sort_noalloc(const int32_t* topk_idx, int64_t N, int32_t k, int64_t M,
                                       int32_t* sorted_expert, int32_t* sorted_slot, int32_t* offsets,
                                       void* stream) {
  const more_status c = dispatch_sort_check(topk_idx, N, k, M, sorted_expert, sorted_slot, offsets);
  if (c != MORE_OK || N == 0) return c;
  if (more_dispatch_workspace_bytes(N, k, M) > kNoAllocScratchBytes) return MORE_ERR_SCRATCH_LIMIT;
  char* ws = (char*)noalloc_scratch();
  if (!ws) return MORE_ERR_HIP;
  return dispatch_sort_run(topk_idx, N, k, M, sorted_expert, sorted_slot, offsets, ws, (hipStream_t)stream);
}

more_status more_topk_merge(int64_t N, int64_t M, int64_t shard_width, int32_t k, more_gate gate,
                            const float* cand_logit, const int32_t* cand_idx, const float* shard_lse,
                            int32_t* topk_idx, float* topk_gate, float* topk_logit, float* lse, void* stream) {
  if (gate != MORE_GATE_TOPK_SOFTMAX && gate != MORE_GATE_FULL_SOFTMAX) return MORE_ERR_BAD_GATE;
  if (N < 0 || N > (1LL << 40) || M < 1 || M > (1 << 24) || shard_width < 1) return MORE_ERR_BAD_SHAPE;
  if (k < 1 || k > MORE_MAX_K || (int64_t)k > shard_width) return MORE_ERR_BAD_K;
  const int64_t G = (M + shard_width - 1) / shard_width;
  if (M - (G - 1) * shard_width < k) return MORE_ERR_BAD_K;   // the last shard holds fewer than k experts
  if (N == 0) return MORE_OK;
  const bool full = gate == MORE_GATE_FULL_SOFTMAX;
  if (!cand_logit || !cand_idx || !topk_idx || !topk_gate || (full && !shard_lse)) return MORE_ERR_NULL_ARG;
  MergeArgs a;
  a.cand_logit = cand_logit;
  a.cand_idx = cand_idx;
  a.shard_lse = shard_lse;
  a.out_idx = topk_idx;
  a.out_gate = topk_gate;
  a.out_logit = topk_logit;
  a.out_lse = full ? lse : nullptr;
  a.N = N;
  a.W = shard_width;
  a.G = (int)G;
  a.k = k;
  return launch_topk_merge(a, full, (hipStream_t)stream) == hipSuccess ? MORE_OK : MORE_ERR_HIP;
}

more_status more_route_fullrank(more_dtype dt, const void* X, int64_t N, int64_t h, const void* W,
                                int64_t M, const float* bias, int32_t k, more_gate gate,
                                int32_t* topk_idx, float* topk_gate, float* topk_logit, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  more_status st = validate(1, dt, X, N, h, W, 0, nullptr, M, bias, k, gate, topk_idx, topk_gate,
                            topk_logit, lse);
  if (st != MORE_OK || N == 0) return st;
  Layout L;
  make_layout(1, dt, h, 0, M, &L);
  hipStream_t s = (hipStream_t)stream;
  if (dt == MORE_DT_BF16 && fr_tiled_supported(h, M, k)) {
    // LDS-tiled MFMA sweep (k <= 8, h a multiple of 64)
    if (!workspace || workspace_bytes < fr_tiled_bytes(h, M) || ((uintptr_t)workspace % kAlign) != 0)
      return MORE_ERR_WORKSPACE;
    return launch_fullrank_tiled((const uint16_t*)X, N, (int)h, (const uint16_t*)W, (int)M, bias, k,
                                 gate == MORE_GATE_FULL_SOFTMAX, topk_idx, topk_gate, topk_logit, lse, workspace,
                                 s) == hipSuccess ? MORE_OK : MORE_ERR_HIP;
  }
  if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace % kAlign) != 0)
    return MORE_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  st = launch_pack(dt, 1, W, nullptr, bias, h, 0, M, L, ws, s);
  if (st != MORE_OK) return st;
  const bool full = gate == MORE_GATE_FULL_SOFTMAX;
  const int kmax = kmax_for(k);
  const int waves = waves_for(kmax);
  FullRankArgs a;
  a.X = X;
  a.N = N;
  a.h = (int)h;
  a.NT = L.NT;
  a.k = k;
  a.KSW = L.ks2;
  a.Wp = ws + L.off_r2p;
  a.biasp = (const float*)(ws + L.off_bias);
  a.perm = (const int*)(ws + L.off_perm);
  a.out_idx = topk_idx;
  a.out_gate = topk_gate;
  a.out_logit = topk_logit;
  a.out_lse = full ? lse : nullptr;
  const int64_t per_block = (int64_t)waves * kTile;
  const dim3 grid((unsigned)((N + per_block - 1) / per_block));
  const size_t shmem = (size_t)waves * log_bytes(kmax);
  hipLaunchKernelGGL(pick_fullrank((int)dt, full, kmax), grid, dim3(64 * waves), shmem, s, a);
  return hipGetLastError() == hipSuccess ? MORE_OK : MORE_ERR_HIP;
}

}  // extern "C"
