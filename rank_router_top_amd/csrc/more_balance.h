// more_balance.h -- balancing statistics of the training forward.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.2.1: Algorithm 2's second sweep recomputes every logit
// tile once the normaliser of each token is known and accumulates the
// column sums of the full softmax, psum_i = sum_n P_{n,i} (eq. 6, 7); the
// Switch loss (eq. 9) needs only psum and f, a bincount of the selected
// indices; App. G.1 defines the normalised entropy of the per-expert counts.
//
// Kernels (all after the routing kernel has written lse, with z of every
// 32-token block still in the token scratch):
//   psum_kernel   recomputes z R2 tile by tile with the MFMA operands swapped
//                 with respect to the routing kernel (z is A, the weights are
//                 B), so a lane holds ONE expert and 16 tokens: the column sum
//                 is 16 in-lane adds, no cross-lane work.  Each wave keeps the
//                 weight operands of its expert tiles in registers for its
//                 whole life and streams z blocks past them; the accumulator
//                 starts at -lse of the token, so exp2((acc + b) log2 e) is P.
//                 Partial sums go to a per-slot row of the workspace (plain
//                 stores: the result does not depend on scheduling).
//   count_kernel  LDS histogram of the selected indices per token slot.
//   colsum_kernel sums the slot rows in a fixed order: psum (by expert index,
//                 via the sweep order) and the counts.
//   stats_kernel  one workgroup: L_bal and H_norm in fp64.
#pragma once
#include "more_device.h"
#include "more_split.h"

namespace more {

constexpr int kBalSlots = 256;     // token slots (rows of partial sums) at most
constexpr int kBalWaves = 8;       // psum_kernel: waves per workgroup
constexpr int kCountBins = 8192;   // count_kernel: LDS bins per workgroup (one expert range)
constexpr int kCountThreads = 256;

// Expert tiles whose weight operands one psum wave keeps in registers.
constexpr int bal_tiles(int r16) { return r16 == 1 ? 16 : r16 == 2 ? 8 : 4; }

struct PsumArgs {
  const void* Z;        // z blocks as written by proj_kernel (bf16 hi, then lo)
  const float* lse;     // N, from the routing kernel
  const void* R2p;      // packed up-projection: tile t at t * R16 * 1024 bytes
  const float* biasp;   // packed bias, accumulator layout, -inf on padding rows
  float* part;          // [slots][Mpad] partial column sums by sweep position
  long long N;
  int NB, NT, G, slots; // token blocks, expert tiles, expert groups, token slots
};

// Grid: slots * G workgroups of 64 * WAVES threads.  Workgroup (s, g) covers
// the token blocks s, s + slots, ... and expert tiles g * WAVES * TW .. +
// WAVES * TW - 1 (wave w: TW consecutive tiles).
template <int R16, int TW, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void psum_kernel(PsumArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = blockIdx.x / a.G, g = blockIdx.x % a.G;
  const int t0 = (g * WAVES + wave) * TW;
  const int hf = lane >> 5;
  const int mpad = a.NT * kTile;
  // weight operands and bias (log2 domain) of this wave's tiles; tiles past NT
  // read zeros and are never stored
  const rsrc_t r2d = make_rsrc(a.R2p, a.NT * R16 * 1024);
  bf16x8 w[TW][R16];
  float bl[TW];
  {
    const int i = lane & 31;
    const int bidx = ((i >> 2) & 1) * 16 + 4 * (i >> 3) + (i & 3);
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      const int t = t0 + u < a.NT ? t0 + u : a.NT - 1;
#pragma unroll
      for (int m = 0; m < R16; ++m) w[u][m] = buf_load(r2d, lane * 16 + m * 1024, t * R16 * 1024);
      bl[u] = a.biasp[t * 32 + bidx] * kLog2e;
    }
  }
  float cs[TW];
#pragma unroll
  for (int u = 0; u < TW; ++u) cs[u] = 0.f;
  // operands of one token block: z (bf16 hi, lo) and lse of token
  // 8q + 4hf + e of the block (register 4q + e).  Two buffers in turn: the
  // next block's loads are issued before the current block is swept, and
  // nothing reads them until its own sweep (no early wait on the queue).
  struct Blk {
    bf16x8 zh[R16], zl[R16];
    float lr[16];
  };
  auto load_blk = [&](long long j, Blk& b) {
    const rsrc_t zd = make_rsrc((const char*)a.Z + (size_t)j * z_block_bytes(R16), z_block_bytes(R16));
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      b.zh[m] = buf_load(zd, lane * 16 + m * 1024, 0);
      b.zl[m] = buf_load(zd, lane * 16 + (R16 + m) * 1024, 0);
    }
    const long long n0 = j * kTile + 4 * hf;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const long long tok = n0 + 8 * (v >> 2) + (v & 3);
      b.lr[v] = a.lse[tok < a.N ? tok : a.N - 1];   // clamped: the row is dropped below
    }
  };
  auto sweep_blk = [&](long long j, const Blk& b) {
    // the block's operands are first touched here, after the loads of the
    // other buffer have been issued (the scheduler may not hoist the uses)
    __builtin_amdgcn_sched_barrier(0);
    // accumulator start -lse; tokens past N start at -inf and add exp2(-inf) = 0
    floatx16 c0;
    const long long n0 = j * kTile + 4 * hf;
#pragma unroll
    for (int v = 0; v < 16; ++v) c0[v] = n0 + 8 * (v >> 2) + (v & 3) < a.N ? -b.lr[v] : -__builtin_inff();
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      floatx16 acc = c0;
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(b.zh[m], w[u][m], acc);
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(b.zl[m], w[u][m], acc);
      float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
      for (int v = 0; v < 16; v += 4) {
        p0 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], kLog2e, bl[u]));
        p1 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v + 1], kLog2e, bl[u]));
        p2 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v + 2], kLog2e, bl[u]));
        p3 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v + 3], kLog2e, bl[u]));
      }
      cs[u] += (p0 + p1) + (p2 + p3);
    }
  };
  // Loads are issued unconditionally (past the last block they re-read the
  // last one and are never swept), so the wait counts stay static.
  Blk b0, b1;
  const long long st = a.slots, last = a.NB - 1;
  long long j = s;
  load_blk(j, b0);   // s < slots <= NB
  for (;; j += 2 * st) {
    load_blk(j + st < last ? j + st : last, b1);
    sweep_blk(j, b0);
    if (j + st >= a.NB) break;
    load_blk(j + 2 * st < last ? j + 2 * st : last, b0);
    sweep_blk(j + st, b1);
    if (j + 2 * st >= a.NB) break;
  }
  // both halves of a lane pair hold the same expert: add them, the low half stores
  float* row = a.part + (size_t)s * mpad;
#pragma unroll
  for (int u = 0; u < TW; ++u) {
    const float tot = cs[u] + partner_f32(cs[u], hf != 0);
    if (hf == 0 && t0 + u < a.NT) row[(t0 + u) * kTile + lane] = tot;
  }
}

struct CountArgs {
  const int* idx;       // N x k selected experts
  int* cpart;           // [slots][M] per-slot counts
  long long N;
  int k, M, NB, slots;
};

struct ColsumArgs {
  const float* part;    // [slots][Mpad]
  const int* cpart;     // [slots][M]
  const int* perm;      // sweep position -> expert (-1 on padding)
  float* psum;          // M
  int* counts;          // M
  int M, Mpad, slots;
};

struct StatsArgs {
  const float* psum;
  const int* counts;
  float* stats;         // [0] L_bal (eq. 9), [1] H_norm (App. G.1)
  long long N;
  int k, M;
};

// Enqueues psum_kernel (instance for r16), count_kernel, colsum_kernel and
// stats_kernel on `stream`.
hipError_t launch_balance(int r16, const PsumArgs& pa, const CountArgs& ca, const ColsumArgs& sa,
                          const StatsArgs& ta, hipStream_t stream);

}  // namespace more
