// more_fullrank_tiled.h -- fused full-rank router as an LDS-tiled MFMA sweep.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", §2 (the standard router: softmax over TopK of l = x W + b) fused
// as in App. H.3 / Fig. 20: the N x M logits stay on chip.  Gates as Fig. 12
// (softmax over the k selected) or eq. (6) with the normaliser of eq. (8).
//
// The full-rank product is a dense contraction (2 N h M flops, K = h), so it
// is tiled like a GEMM.  One workgroup (8 waves) owns 256 tokens and sweeps
// the experts in slabs of 256; over K it streams 32-wide chunks of its X block
// (16 KiB) and of the slab's weights (16 KiB) straight from global memory into
// LDS rings.  Wave (wt, we) accumulates tokens 64 wt .. +64 (two 32-token
// groups) against experts 128 we .. +128 of the slab (four 32-expert tiles):
// eight 32x32 fp32 accumulators, 16 v_mfma_f32_32x32x16_bf16 per chunk
// against 12 LDS operand reads.  The square tile keeps the operand bytes per
// flop at their minimum for the accumulators a CU holds.  At the end of a
// slab every lane (token column, half hf) folds its 16 logits per tile into a
// register top-k list (value desc, expert asc) and, for eq. (6), the running
// maximum and normaliser of eq. (8); at the end of the sweep the 4 lists of
// each token (2 expert halves x 2 lane halves) are merged through LDS.
//
// Weights are packed per call by fr_pack_kernel in natural expert order:
// unit (slab, chunk, tile, kstep, lane) holds the 8 bf16 W[k][j] of the
// 32x32x16 A operand, j = 256 slab + 32 tile + lane % 32,
// k = 32 chunk + 16 kstep + 8 (lane / 32) + e; rows past M and columns past h
// are zero, and the bias in accumulator layout is -inf past M.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace more {

constexpr int kFrWaves = 8;          // waves per workgroup
constexpr int kFrTokens = 256;       // tokens per workgroup
constexpr int kFrSlab = 256;         // experts per slab
constexpr int kFrChunk = 32;         // K per LDS chunk (two MFMA K-steps)
constexpr int kFrKmax = 8;           // largest k of the tiled kernel

struct FrTiledArgs {
  const uint16_t* X;      // N x h bf16
  const uint16_t* Wq;     // packed weights (see above)
  const float* biasq;     // [nslab][8][2][16]
  int* out_idx;
  float* out_gate;
  float* out_logit;
  float* out_lse;
  long long N;
  int h, nslab, k;
};

// Bytes of packed weights + bias for (h, M); h must be a multiple of 2 kFrChunk.
inline size_t fr_tiled_bytes(long long h, long long M) {
  const long long nslab = (M + kFrSlab - 1) / kFrSlab;
  return (size_t)(nslab * kFrSlab * h * 2) + (size_t)(nslab * kFrSlab * 4);
}

// Whether the tiled kernel covers the call (bf16 only; the chunk count
// (M / kFrSlab) (h / kFrChunk) stays well inside int).
inline bool fr_tiled_supported(long long h, long long M, int k) {
  return h % (2 * kFrChunk) == 0 && k <= kFrKmax && M >= 1 &&
         ((M + kFrSlab - 1) / kFrSlab) * (h / kFrChunk) < (1LL << 30);
}

// Packs W (h x M bf16) and the bias into `ws` (fr_tiled_bytes(h, M) bytes,
// 256-byte aligned) and launches the tiled kernel on `stream`.
hipError_t launch_fullrank_tiled(const uint16_t* X, long long N, int h, const uint16_t* W, int M,
                                 const float* bias, int k, bool full, int* out_idx, float* out_gate,
                                 float* out_logit, float* out_lse, void* ws, hipStream_t stream);

}  // namespace more
