// more_backward.h -- backward pass of the low-rank router with recompute.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.2.2 (eq. 10-12) and Algorithm 3.  With the selection idx
// fixed, incoming gradients tvbar (N x k, on the selected logits) and pbar (M,
// on psum) and the forward's lse, per token n:
//   g_n = sum_i pbar_i P_{n,i},   P = exp(l - lse)
//   ybar_{n,j} = P_{n,j} (pbar_j - g_n) + [tvbar at the selected experts]
//   zbar = ybar R2^T,  xbar = zbar R1^T,
// and over tokens R2bar = z^T ybar, R1bar = x^T zbar, bbar = sum_n ybar.
// (Convention: R1 is h x r, R2 is r x M, l = (x R1) R2 + b.)
//
// Kernels (in k_backward.hip; after proj_kernel has written z of every
// 32-token block):
//   bwd_pack_kernel  per call: pbar in the accumulator layout and by sweep
//                    position, R2 as the A operand of zbar^T = R2 ybar^T
//                    (K = the 32 experts of a tile in the order a token
//                    lane holds them), R2 expert-major (rows of 32), and the
//                    expert -> position map.
//   bwd_tok_kernel   token-stationary (one wave per 32-token block, lane =
//                    token as in the routing kernel): sweep 1 over every tile
//                    gives g; sweep 2 recomputes P and feeds the dense part of
//                    ybar straight into MFMAs for zbar^T (ybar in the
//                    accumulator layout is already a B operand).  The sparse
//                    part adds tvbar times R2's selected columns.  Writes g,
//                    zbar and z (fp32 rows of 32).
//   bwd_exp_kernel   expert-stationary (lane = expert, as psum_kernel): each
//                    wave keeps 2 tiles' operands and their R2bar partials
//                    (32 x 32 fp32 each) in registers; the workgroup stages
//                    each token block's operands in LDS once, one block ahead;
//                    each wave recomputes P, adds tvbar through a per-wave
//                    LDS tile, and accumulates R2bar += z^T ybar (MFMA) and
//                    bbar (in-lane sums).
//   bwd_x_kernel     streams X once: per 32-token block and 32-column h tile,
//                    xbar = zbar R1^T (MFMA, stored bf16) and the R1bar^T
//                    partial += zbar^T X (MFMA, X from 2-byte column loads).
//   bwd_reduce_kernel  fixed-order sums of the per-slot partials into
//                    R2bar (expert order), bbar and R1bar.
#pragma once
#include <algorithm>

#include "more_device.h"
#include "more_split.h"

namespace more {

constexpr int kBwdSlots = 64;      // token slots of the expert- and h-stationary kernels
constexpr int kBwdTokWaves = 8;    // bwd_tok_kernel waves per workgroup
constexpr int kBwdExpWaves = 8;    // bwd_exp_kernel waves per workgroup (two per SIMD)
constexpr int kBwdExpTiles = 2;    // expert tiles per bwd_exp wave
constexpr int kBwdXWaves = 4;
constexpr int kBwdXTiles = 2;      // h tiles (32 columns) per bwd_x wave
constexpr int kBwdRow = 32;        // row stride of z, zbar (ranks padded to 32)

struct BwdArgs {
  // forward pieces (packed workspace, token scratch)
  const void* Z;            // z blocks (bf16 hi, lo) from proj_kernel
  const float* lse;         // N (forward output)
  const void* R2p;          // logits A operand, tile t at t * R16 * 1024 bytes
  const float* biasp;       // [NT][2][16] accumulator layout, -inf on padding
  const int* perm;          // position -> expert (-1 on padding)
  // user inputs
  const uint16_t* X;        // N x h bf16
  const uint16_t* R1;       // h x r bf16
  const uint16_t* R2;       // r x M bf16
  const int* idx;           // N x k
  const float* tv;          // N x k
  const float* pbar;        // M or null
  // per-call packing (bwd_pack_kernel)
  float* pbq;               // [NT][2][16]
  float* pbpos;             // [Mpad]
  uint16_t* R2b;            // [NT][2][64][8]
  uint16_t* R2t;            // [M][32]
  int* invpos;              // [M]
  // intermediates
  int* selpos;              // N x k: sweep position * 32 + token within its block
  float* g;                 // N
  float* zbar;              // N x 32
  float* zrm;               // N x 32
  // partials and outputs
  float* r2part;            // [slotsE][32][Mpad]
  float* bpart;             // [slotsE][Mpad]
  float* r1part;            // [slotsX][h][32]
  uint16_t* xbar;           // N x h bf16
  float* r1grad;            // h x r
  float* r2grad;            // r x M
  float* bgrad;             // M or null
  long long N;
  int h, r, M, k, NT, NB, slotsE, GE, slotsX, GX;
};

// Enqueues bwd_pack_kernel, bwd_tok_kernel, bwd_exp_kernel, bwd_x_kernel and
// bwd_reduce_kernel (instances for r16) on `stream`; the projection of z runs
// before, from the caller.
hipError_t launch_backward(int r16, const BwdArgs& a, size_t tok_lds, int cus, hipStream_t stream);

}  // namespace more
