// more_pack.h -- per-call preparation: expert sweep order and MFMA operand packing.
//
// The fused kernels read every weight operand with one 16-byte load per lane
// in the exact register layout the MFMA wants, from a packed copy in the
// caller's workspace (L2-resident: 128 KiB + 256 KiB at h=2048, r=32, M=4096).
//
// Sweep order.  Without a bias the experts are swept in index order.  With a
// bias (M <= 16384) they are swept by bias descending (ties by index), as
// sorted by more_order.h before this kernel runs: experts with a large bias tend to end
// in the top-k, so the running k-th value rises early and fewer later logits
// pass the filter.  The selected set and its order do not depend on the sweep
// order (ties are resolved by expert index at the end), so this is purely a
// speed choice.
#pragma once
#include "more_device.h"

namespace more {

// Position p of the sweep holds expert perm[p] (perm[p] = -1 on the padding
// positions M..M_pad-1).  Row i of tile t is position 32t + i.  For a lane of
// half hf, accumulator register v holds row 8*(v>>2) + 4*hf + (v&3).
__host__ __device__ inline int acc_row(int v, int hf) { return 8 * (v >> 2) + 4 * hf + (v & 3); }

struct PackArgs {
  // inputs
  const void* R1;     // h x r (bf16 bits or fp32)
  const void* R2;     // r x M, or W (h x M) for full rank
  const float* bias;  // M or null
  int h, r, M, Mpad, NT;
  int kdim;           // contraction length of the second product: r (low rank) or h (full rank)
  int ksteps2;        // MFMA K-steps of the second product
  int ksteps1, rb;    // first product: K-steps over h and 32-row blocks of z (low rank only)
  int natural_k;      // 1: second-product K rows in memory order (full rank: the X operand)
  int rank_blocks;    // blocks packing the second product's operands (64 sweep positions each)
  int r1_blocks;      // blocks packing R1
  int ksq, r16;       // producer layout of R1: 32-column K-steps (padded) and 16-rank blocks
  int r1q_blocks;     // blocks packing R1q (0: not wanted)
  // outputs (workspace)
  void* R1p;
  void* R1q;          // [ksq][r16][64][8] bf16, A operand of v_mfma_f32_16x16x32_bf16 (R1^T block)
  void* R2p;
  float* biasp;       // [NT][2][16] fp32, accumulator layout (fp32 kernels)
  uint32_t* biasq;    // [NT][64] bf16 pairs (hi, lo) as an MFMA A operand (bf16 kernels)
  int* perm;          // [Mpad]: read (with a bias: sorted beforehand) or written (without)
  int sorted;         // 1: perm was written by the order kernels (bias-descending order)
  int* status;        // the routing calls' stall word: cleared (null: left alone)
  int* seed;          // seed-pass length of the LDS-ring sweep (tiles), written (null: left alone)
  int seed_tiles;
};

// Element type helpers.
template <int DT> struct Elem;
template <> struct Elem<0> { typedef uint16_t T; };   // bf16 bits
template <> struct Elem<1> { typedef float T; };

// K index (row of R2 / W) carried by element e of K-step m for lane half hf.
// Low rank (natural = 0), the rows of z as the first product left them:
//  bf16 (8 elements per lane): rho = 16m + 8(e>>2) + 4hf + (e&3), which is
//    accumulator register v = 8*(m&1) + e of 32-row block m>>1, so z feeds
//    the second MFMA without any shuffle.
//  fp32 (1 element per lane, K=2): rho = 32(m>>4) + acc_row(m & 15, hf).
// Full rank (natural = 1), the memory order of an X row, which each lane loads
// as consecutive elements: 16m + 8hf + e (bf16) or 2m + hf (fp32).
template <int DT>
__host__ __device__ inline int k_row(int m, int e, int hf, int natural) {
  if (natural) return (DT == 0) ? 16 * m + 8 * hf + e : 2 * m + hf;
  if (DT == 0) return 16 * m + 8 * (e >> 2) + 4 * hf + (e & 3);
  return 32 * (m >> 4) + acc_row(m & 15, hf);
}

template <int DT>
__global__ __launch_bounds__(1024) void pack_kernel(PackArgs a) {
  typedef typename Elem<DT>::T T;
  constexpr int EPL = (DT == 0) ? 8 : 1;          // elements per lane per K-step
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && tid == 0) {
    if (a.status) *a.status = 0;
    if (a.seed) *a.seed = a.seed_tiles;
  }
  if ((int)blockIdx.x < a.rank_blocks) {
    // ---- sweep position pos holds expert j = perm[pos] (sorted by
    // order kernels with a bias; index order otherwise); padding last
    const int jl = tid & 63, slice = tid >> 6;   // 64 positions x 16 slices
    // Mpad is a multiple of 64: every position of the block is real
    const int pos = blockIdx.x * 64 + jl;
    const int j = a.sorted ? a.perm[pos] : (pos < a.M ? pos : -1);
    const int t = pos >> 5, i = pos & 31;
    const T* B = (const T*)a.R2;
    T* Bp = (T*)a.R2p;
    // gather column j of R2 (or W) into the packed tile at row i
    for (int w = slice; w < a.ksteps2 * 2 * EPL; w += 16) {
      const int m = w / (2 * EPL), hf = (w / EPL) & 1, e = w % EPL;
      const int kr = k_row<DT>(m, e, hf, a.natural_k);
      T val = 0;
      if (j >= 0 && kr < a.kdim) val = B[(size_t)kr * a.M + j];
      Bp[(((size_t)t * a.ksteps2 + m) * kWave + i + 32 * hf) * EPL + e] = val;
    }
    if (slice == 0) {
      if (!a.sorted) a.perm[pos] = j;
      const int hf = (i >> 2) & 1, v = 4 * (i >> 3) + (i & 3);
      const float bv = (j >= 0) ? (a.bias ? a.bias[j] : 0.f) : -__builtin_inff();
      a.biasp[(t * 2 + hf) * 16 + v] = bv;
      if (a.biasq) {
        // bias of row i as bf16 hi + lo in K-slots 0 and 1 of lane i (lanes 32..63
        // carry zeros): one MFMA against a ones operand adds hi + lo to every token.
        const bf16 bh = (bf16)bv;
        const float rest = (j >= 0) ? bv - (float)bh : 0.f;
        const bf16 bl = (bf16)rest;
        a.biasq[(size_t)t * kWave + i] =
            (uint32_t)__builtin_bit_cast(uint16_t, bh) | ((uint32_t)__builtin_bit_cast(uint16_t, bl) << 16);
        a.biasq[(size_t)t * kWave + 32 + i] = 0u;
      }
    }
    return;
  }
  if ((int)blockIdx.x >= a.rank_blocks + a.r1_blocks) {
    // ---- R1q (bf16, low rank): entry (s, rb, lane) holds rows 32s + 8(lane/16) .. +7
    // of R1, column 16rb + lane%16 -- lane l of the A operand is row l%16 of the
    // 16 x 32 block R1^T[16rb.., 32s..], K slots 8(l/16) .. +7.
    if constexpr (DT == 0) {
      const int gq = ((int)blockIdx.x - a.rank_blocks - a.r1_blocks) * 1024 + tid;
      if (gq >= a.ksq * a.r16 * kWave) return;
      const int lane = gq % kWave, srb = gq / kWave;
      const int rbk = srb % a.r16, s = srb / a.r16;
      const int col = 16 * rbk + (lane & 15);
      const uint16_t* A = (const uint16_t*)a.R1;
      uint16_t* Aq = (uint16_t*)a.R1q;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int hrow = 32 * s + 8 * (lane >> 4) + e;
        Aq[(size_t)gq * 8 + e] = (hrow < a.h && col < a.r) ? A[(size_t)hrow * a.r + col] : (uint16_t)0;
      }
    }
    return;
  }
  // ---- R1 packing (low rank only): entry (s, b, lane) holds the A operand of
  // K-step s for 32-row block b of z.
  const int gidx = ((int)blockIdx.x - a.rank_blocks) * 1024 + tid;
  const int total = a.ksteps1 * a.rb * kWave;
  if (gidx >= total) return;
  const int lane = gidx % kWave, sb = gidx / kWave;
  const int b = sb % a.rb, s = sb / a.rb;
  const int hf = lane >> 5, col = 32 * b + (lane & 31);
  const T* A = (const T*)a.R1;
  T* Ap = (T*)a.R1p;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int hrow = (DT == 0) ? 16 * s + 8 * hf + e : 2 * s + hf;
    T val = 0;
    if (hrow < a.h && col < a.r) val = A[(size_t)hrow * a.r + col];
    Ap[(size_t)gidx * EPL + e] = val;
  }
}

}  // namespace more
