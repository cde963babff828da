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
//                 whole life; the workgroup stages each token block's z,
//                 scaled by log2 e, in LDS, and the bias factors out of the
//                 exponentials (see the kernel).  Partial sums go to a
//                 per-slot row of the workspace (plain stores: the result
//                 does not depend on scheduling).
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
//
// All waves of a workgroup walk the same token blocks, so each block's
// operands are prepared once, in LDS: z scaled by log2 e and split again into
// bf16 hi + lo (so the MFMAs produce logits in log2 units), and -lse log2 e
// per token; the next block's raw z and lse are loaded before the current
// block is swept.  With the accumulator starting at -lse log2 e + B_w (B_w =
// the largest biased log2 scale among the wave's experts), one tile's column
// sum is exp2(b_e log2 e - B_w) * sum_v exp2(acc_v): 16 exp2 and 16 adds, the
// bias factored out of the exponentials.  Every acc_v <= B_w - b_e log2 e, so
// nothing overflows while the wave's bias spread stays below 100 log2 units;
// beyond that the wave takes the unfactored form, exp2(acc_v + b_e log2 e).
template <int R16, int TW, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void psum_kernel(PsumArgs a) {
  constexpr int ZCH = R16 * 64;            // 16-byte chunks of z hi (and of z lo) per block
  __shared__ __align__(16) u32x4 zs[2][2 * ZCH];
  __shared__ __align__(16) float ls[2][kTile];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // B_w and the wave's bias spread (finite entries; padding rows are -inf)
  float bmax = -__builtin_inff(), bmin = __builtin_inff();
#pragma unroll
  for (int u = 0; u < TW; ++u)
    if (bl[u] > -__builtin_inff()) {
      bmax = fmaxf(bmax, bl[u]);
      bmin = fminf(bmin, bl[u]);
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    bmax = fmaxf(bmax, __shfl_xor(bmax, o));
    bmin = fminf(bmin, __shfl_xor(bmin, o));
  }
  const bool factored = !(bmax > -__builtin_inff()) || bmax - bmin < 100.f;
  const float Bw = bmax > -__builtin_inff() ? bmax : 0.f;
  float eb[TW];
#pragma unroll
  for (int u = 0; u < TW; ++u) eb[u] = __builtin_amdgcn_exp2f(bl[u] - Bw);   // 0 on padding rows
  float cs[TW];
#pragma unroll
  for (int u = 0; u < TW; ++u) cs[u] = 0.f;
  // staging of one block: threads < ZCH take one hi and one lo chunk (8 ranks
  // each), threads < 32 one lse
  struct Pre {
    u32x4 h, l;
    float lse;
  };
  auto fetch = [&](long long j, Pre& P) {
    const u32x4* zb = (const u32x4*)((const char*)a.Z + (size_t)j * z_block_bytes(R16));
    const int c = tid < ZCH ? tid : 0;
    P.h = zb[c];
    P.l = zb[ZCH + c];
    const long long tk = j * kTile + (tid & 31);
    P.lse = a.lse[tk < a.N ? tk : a.N - 1];
  };
  auto stage = [&](long long j, const Pre& P, int buf) {
    if (tid < ZCH) {
      const bf16x8 hv = __builtin_bit_cast(bf16x8, P.h), lv = __builtin_bit_cast(bf16x8, P.l);
      bf16x8 h2, l2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = ((float)hv[e] + (float)lv[e]) * kLog2e;
        const bf16 hh = (bf16)x;
        h2[e] = hh;
        l2[e] = (bf16)(x - (float)hh);
      }
      zs[buf][tid] = __builtin_bit_cast(u32x4, h2);
      zs[buf][ZCH + tid] = __builtin_bit_cast(u32x4, l2);
    }
    if (tid < kTile) {
      const long long tk = j * kTile + tid;
      ls[buf][tid] = tk < a.N ? -P.lse * kLog2e : -__builtin_inff();   // tokens past N: P = 0
    }
  };
  auto sweep = [&](int buf) {
    bf16x8 zh[R16], zl[R16];
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      zh[m] = __builtin_bit_cast(bf16x8, zs[buf][m * 64 + lane]);
      zl[m] = __builtin_bit_cast(bf16x8, zs[buf][ZCH + m * 64 + lane]);
    }
    // accumulator start for token 8q + 4hf + e of the block (register 4q + e)
    floatx16 c0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *(const float4*)(&ls[buf][8 * q + 4 * hf]);
      c0[4 * q] = v.x;
      c0[4 * q + 1] = v.y;
      c0[4 * q + 2] = v.z;
      c0[4 * q + 3] = v.w;
    }
    if (factored) {
#pragma unroll
      for (int v = 0; v < 16; ++v) c0[v] += Bw;
#pragma unroll
      for (int u = 0; u < TW; ++u) {
        floatx16 acc = c0;
#pragma unroll
        for (int m = 0; m < R16; ++m) acc = mfma_bf16(zh[m], w[u][m], acc);
#pragma unroll
        for (int m = 0; m < R16; ++m) acc = mfma_bf16(zl[m], w[u][m], acc);
        float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
        for (int v = 0; v < 16; v += 4) {
          p0 += __builtin_amdgcn_exp2f(acc[v]);
          p1 += __builtin_amdgcn_exp2f(acc[v + 1]);
          p2 += __builtin_amdgcn_exp2f(acc[v + 2]);
          p3 += __builtin_amdgcn_exp2f(acc[v + 3]);
        }
        cs[u] = __builtin_fmaf(eb[u], (p0 + p1) + (p2 + p3), cs[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < TW; ++u) {
        floatx16 acc = c0;
#pragma unroll
        for (int m = 0; m < R16; ++m) acc = mfma_bf16(zh[m], w[u][m], acc);
#pragma unroll
        for (int m = 0; m < R16; ++m) acc = mfma_bf16(zl[m], w[u][m], acc);
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          p0 += __builtin_amdgcn_exp2f(acc[v] + bl[u]);
          p1 += __builtin_amdgcn_exp2f(acc[v + 1] + bl[u]);
        }
        cs[u] += p0 + p1;
      }
    }
  };
  Pre P;
  long long j = s;   // s < slots <= NB
  fetch(j, P);
  stage(j, P, 0);
  __syncthreads();
  int cur = 0;
  for (; j < a.NB; j += a.slots) {
    const bool more = j + a.slots < a.NB;
    if (more) fetch(j + a.slots, P);
    sweep(cur);
    if (more) stage(j + a.slots, P, cur ^ 1);
    __syncthreads();   // the next buffer is complete; the current one is free again
    cur ^= 1;
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
