// Fused full-rank router, LDS-tiled MFMA form: weight packing, kernel, launch.
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", §2 (standard router), App. H.3 / Fig. 20 (fused, no logits in
// memory), Fig. 12 and eq. (6) / (8) (gates).
#include "more_device.h"
#include "more_fullrank_tiled.h"

namespace more {

namespace {
constexpr int kFrThreads = 64 * kFrWaves;
constexpr int kFrXBytes = kFrTokens * kFrChunk * 2;        // X chunk of the block
constexpr int kFrWBytes = kFrSlab * kFrChunk * 2;          // weight chunk of the slab
constexpr int kFrBBytes = kFrSlab * 4;                     // the slab's bias
constexpr int kFrWBuf = kFrWBytes + 2 * kFrBBytes;         // one weight + bias buffer (bias twice: see issue_w)
constexpr int kFrUnitsW = kFrWBytes / 16;                  // 16-byte units of a weight chunk
constexpr int kFrTiles = kFrSlab / 32;                     // 32-expert tiles of a slab
constexpr int kFrLists = 2 * 2;                            // lists per token: 2 expert halves x 2 lane halves
// Weight chunks are loaded 2 chunks ahead (3 buffers); X chunks, which miss
// L2 (every slab re-reads the block), 5 chunks ahead (6 buffers).
constexpr int kFrWBufs = 3;
constexpr int kFrXBufs = 6;
constexpr int kFrLds = kFrWBufs * kFrWBuf + kFrXBufs * kFrXBytes;
static_assert(kFrLds <= 160 * 1024, "LDS of one workgroup");
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): wait until at most 5 / 3 / 0 vector-memory operations
// of this wave are outstanding, nothing else.  Per chunk a lane issues 2 X
// loads and 3 weight + bias loads.
constexpr int kVmcnt5 = 0x0f70 | 5;
constexpr int kVmcnt3 = 0x0f70 | 3;
constexpr int kVmcnt0 = 0x0f70;
static_assert(kFrTokens * kFrChunk * 2 == kFrWaves * 2 * kWave * 16, "two X operand blocks per wave");
static_assert(kFrUnitsW % kFrThreads == 0, "whole weight units per thread");
static_assert(kFrSlab == 4 * kWave && kFrWaves == 8, "waves 0-3 load the bias, 4-7 a copy");
static_assert(kFrTokens * kFrLists * (kFrKmax + 1) * 8 <= kFrLds, "merge area fits the operand buffers");
static_assert(kFrTokens == kFrWaves * 32 && kFrSlab == 2 * 4 * 32, "wave (w % 4, w / 4): 2 token groups x 4 tiles");
}  // namespace

// Global -> LDS load of `bytes` (16 or 4) per lane: lane l's bytes land at
// LDS byte address lds + l * bytes (lds wave-uniform, through M0).  Written as
// inline assembly so that the compiler does not order LDS reads of the other
// buffers behind it (it cannot tell the buffers apart and would wait for every
// load in flight); the kernel waits for these loads itself (s_waitcnt vmcnt)
// before the barrier that publishes a chunk.  No register is written.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is reserved; it is named to state that it changes
__device__ __forceinline__ void fr_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void fr_dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// Publish a chunk: wait for this wave's loads of it (VMCNT_IMM lets the loads
// of the next chunk stay in flight), then the workgroup barrier.  The empty asm
// statements keep the compiler from moving LDS accesses across the barrier.
template <int VMCNT_IMM>
__device__ __forceinline__ void fr_publish() {
  __builtin_amdgcn_s_waitcnt(VMCNT_IMM);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One thread per 16-byte unit of packed weights; the first nslab * 512 threads
// also write the bias in accumulator layout (lane half hf, register v holds
// row 8 (v / 4) + 4 hf + v % 4 of the 32-expert tile).
__global__ __launch_bounds__(256) void fr_pack_kernel(const uint16_t* __restrict__ W, const float* __restrict__ bias,
                                                      int h, int M, int nslab, uint16_t* __restrict__ Wq,
                                                      float* __restrict__ biasq) {
  const long long NC = h / kFrChunk;
  const long long units = (long long)nslab * NC * kFrUnitsW;
  const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
  if (u < units) {
    const int lane = (int)(u % 64), s = (int)((u / 64) % 2), t = (int)((u / 128) % kFrTiles);
    const long long c = (u / kFrUnitsW) % NC, slab = u / (kFrUnitsW * NC);
    const long long j = slab * kFrSlab + t * 32 + (lane & 31);
    const long long k0 = c * kFrChunk + 16 * s + 8 * (lane >> 5);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t lo = j < M ? W[(k0 + e) * M + j] : 0u;
      const uint32_t hi = j < M ? W[(k0 + e + 1) * M + j] : 0u;
      w[e / 2] = lo | (hi << 16);
    }
    *(uint4*)(Wq + u * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (u < (long long)nslab * kFrSlab) {
    const int v = (int)(u % 16), hf = (int)((u / 16) % 2), t = (int)((u / 32) % kFrTiles);
    const long long slab = u / kFrSlab;
    const long long j = slab * kFrSlab + t * 32 + 8 * (v / 4) + 4 * hf + v % 4;
    biasq[u] = j < M ? (bias ? bias[j] : 0.f) : -__builtin_inff();
  }
}

// Insert x (sweep position pos, larger than every position already held)
// into the descending list T / P; equal values keep the earlier entry.
template <int K>
__device__ __forceinline__ void fr_insert(float (&T)[K], int (&P)[K], float x, int pos) {
#pragma unroll
  for (int j = K - 1; j >= 1; --j) {
    const bool cj = x > T[j], cm = x > T[j - 1];
    T[j] = cm ? T[j - 1] : (cj ? x : T[j]);
    P[j] = cm ? P[j - 1] : (cj ? pos : P[j]);
  }
  if (x > T[0]) {
    T[0] = x;
    P[0] = pos;
  }
}

// Fold one 32-expert tile of logits (this lane's 16: rows 8 (v / 4) + 4 hf +
// v % 4, sweep positions pb + 8 (v / 4) + v % 4) into the lane's list and,
// for eq. (6), into the running maximum m and normaliser z of eq. (8).  A value
// below the partner half's k-th, or not above this lane's own k-th (which
// came earlier), cannot be among the token's top k.
template <int K, bool FULL>
__device__ __forceinline__ void fr_fold(float (&T)[K], int (&P)[K], float& m, float& z, const floatx16& v, int pb,
                                        bool hi) {
  float g4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) g4[q] = fmaxf(fmaxf(v[4 * q], v[4 * q + 1]), fmaxf(v[4 * q + 2], v[4 * q + 3]));
  const float tmax = fmaxf(fmaxf(g4[0], g4[1]), fmaxf(g4[2], g4[3]));
  if (FULL) {
    const float mn = fmaxf(m, tmax);
    const float mb = mn * kLog2e;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += __builtin_amdgcn_exp2f(__builtin_fmaf(v[e], kLog2e, -mb));
    z = z * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + s;
    m = mn;
  }
  const float thr_p = partner_f32(T[K - 1], hi);
  const float thr = fmaxf(T[K - 1], thr_p);
  if (any_lane(tmax >= thr)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (any_lane(g4[q] >= thr)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = v[4 * q + e];
          if (x > T[K - 1] && x >= thr_p) fr_insert<K>(T, P, x, pb + 8 * q + e);
        }
      }
    }
  }
}

template <bool FULL>
__global__ __launch_bounds__(kFrThreads) void fr_tiled_kernel(FrTiledArgs a) {
  constexpr int K = kFrKmax;
  __shared__ __align__(16) char smem[kFrLds];   // [3 weight + bias buffers][6 X buffers]
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = w & 3, we = w >> 2;
  const bool hi = lane >= 32;
  const int hf = hi ? 1 : 0, col = lane & 31;
  const long long tb0 = (long long)blockIdx.x * kFrTokens;
  const int NC = a.h / kFrChunk;   // even: h is a multiple of 2 kFrChunk
  const int Q = a.nslab * NC;

  // Loads go straight from global memory into LDS (16 bytes per lane; the
  // destination of a wave's load is 64 consecutive 16-byte slots): wave w
  // fills the X operand blocks (group w, K-steps 0 and 1) of the chunk, two
  // 1 KiB runs of the weight chunk and 64 bias values (waves 4-7 load a copy,
  // so that every wave issues the same loads).  Rows past N read row N - 1:
  // their logits are never stored.
  const long long xrow = tb0 + w * kTile + col;
  const uint16_t* xsrc = a.X + (xrow < a.N ? xrow : a.N - 1) * (long long)a.h + 8 * hf;
  const uint32_t smem0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  auto issue_x = [&](int q) {
    const int c = q % NC;
    const uint32_t base = __builtin_amdgcn_readfirstlane(smem0 + (uint32_t)(kFrWBufs * kFrWBuf + (q % kFrXBufs) * kFrXBytes));
    fr_dma16(xsrc + (long long)c * kFrChunk, base + (2 * w + 0) * kWave * 16);
    fr_dma16(xsrc + (long long)c * kFrChunk + 16, base + (2 * w + 1) * kWave * 16);
  };
  auto issue_w = [&](int q) {
    const int slab = q / NC;
    const uint32_t base = __builtin_amdgcn_readfirstlane(smem0 + (uint32_t)((q % kFrWBufs) * kFrWBuf));
    const u32x4* ws = (const u32x4*)a.Wq + (long long)q * kFrUnitsW + w * kWave + lane;
#pragma unroll
    for (int i = 0; i < kFrUnitsW / kFrThreads; ++i)
      fr_dma16(ws + i * kFrThreads, base + (i * kFrThreads + w * kWave) * 16);
    fr_dma4(a.biasq + (long long)slab * kFrSlab + (w & 3) * kWave + lane,
            base + kFrWBytes + (w >> 2) * kFrBBytes + (w & 3) * kWave * 4);
  };

  floatx16 acc[2][4];
  auto reset = [&](int buf) {
    const float* bs = (const float*)(smem + buf * kFrWBuf + kFrWBytes);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const floatx16 bv = *(const floatx16*)(bs + ((4 * we + t) * 2 + hf) * 16);
      acc[0][t] = bv;
      acc[1][t] = bv;
    }
  };
  // One chunk: the 12 operand reads, then the 16 MFMAs with the loads of later
  // chunks (X(qx): 2, W(qw): 3, in that order) spread between them, so that a
  // wave never issues a burst of loads while its MFMAs wait.
  auto compute = [&](int wbuf, int xbuf, int qx, int qw) {
    const bf16x8* xs = (const bf16x8*)(smem + kFrWBufs * kFrWBuf + xbuf * kFrXBytes);
    const bf16x8* ws = (const bf16x8*)(smem + wbuf * kFrWBuf);
    bf16x8 bo[2][2], ao[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bo[s][0] = xs[((2 * wt + 0) * 2 + s) * kWave + lane];
      bo[s][1] = xs[((2 * wt + 1) * 2 + s) * kWave + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) ao[s][t] = ws[((4 * we + t) * 2 + s) * kWave + lane];
    }
    const bool dox = qx < Q, dow = qw < Q;
    const uint32_t xl = __builtin_amdgcn_readfirstlane(smem0 + (uint32_t)(kFrWBufs * kFrWBuf + (qx % kFrXBufs) * kFrXBytes)) +
                        2 * w * kWave * 16;
    const uint16_t* xg = xsrc + (long long)(qx % NC) * kFrChunk;
    const uint32_t wb = __builtin_amdgcn_readfirstlane(smem0 + (uint32_t)((qw % kFrWBufs) * kFrWBuf));
    const u32x4* wg = (const u32x4*)a.Wq + (long long)qw * kFrUnitsW + w * kWave + lane;
    const float* bg = a.biasq + (long long)(qw / NC) * kFrSlab + (w & 3) * kWave + lane;
    static_assert(kFrUnitsW / kFrThreads == 2, "two weight loads per lane and chunk");
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int s = m >> 3, t = (m >> 1) & 3, g = m & 1;
      acc[g][t] = mfma_bf16(ao[s][t], bo[s][g], acc[g][t]);
      if (m == 1 || m == 4 || m == 7 || m == 10 || m == 13) {
        __builtin_amdgcn_sched_barrier(0);
        if (m == 1 && dox) fr_dma16(xg, xl);
        if (m == 4 && dox) fr_dma16(xg + 16, xl + kWave * 16);
        if (m == 7 && dow) fr_dma16(wg, wb + w * kWave * 16);
        if (m == 10 && dow) fr_dma16(wg + kFrThreads, wb + (kFrThreads + w * kWave) * 16);
        if (m == 13 && dow) fr_dma4(bg, wb + kFrWBytes + (w >> 2) * kFrBBytes + (w & 3) * kWave * 4);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // per token group: the lane's top-k list over its half of this wave's
  // experts (+inf fillers above the k real slots when k < K), and eq. (8)
  float T[2][K];
  int P[2][K];
  float mr[2], zr[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      T[g][j] = (j < K - a.k) ? __builtin_inff() : kLowest;
      P[g][j] = -1;
    }
    mr[g] = kLowest * 0.25f;
    zr[g] = 0.f;
  }
  auto fold = [&](int slab) {
    const int pb = slab * kFrSlab + 4 * we * kTile + 4 * hf;
    fr_fold<K, FULL>(T[0], P[0], mr[0], zr[0], acc[0][0], pb + 0 * kTile, hi);
    fr_fold<K, FULL>(T[0], P[0], mr[0], zr[0], acc[0][1], pb + 1 * kTile, hi);
    fr_fold<K, FULL>(T[0], P[0], mr[0], zr[0], acc[0][2], pb + 2 * kTile, hi);
    fr_fold<K, FULL>(T[0], P[0], mr[0], zr[0], acc[0][3], pb + 3 * kTile, hi);
    fr_fold<K, FULL>(T[1], P[1], mr[1], zr[1], acc[1][0], pb + 0 * kTile, hi);
    fr_fold<K, FULL>(T[1], P[1], mr[1], zr[1], acc[1][1], pb + 1 * kTile, hi);
    fr_fold<K, FULL>(T[1], P[1], mr[1], zr[1], acc[1][2], pb + 2 * kTile, hi);
    fr_fold<K, FULL>(T[1], P[1], mr[1], zr[1], acc[1][3], pb + 3 * kTile, hi);
  };
  // One barrier per chunk.  Loads are issued in the order X(0), W(0), X(1..4),
  // W(1), then per chunk q: X(q + 5), W(q + 2); so X(q) always precedes W(q),
  // and before chunk q at most the loads of the previous iteration (X(q + 4):
  // 2, W(q + 1): 3) may still fly.  The wait + barrier make chunk q visible
  // and free the buffers of chunk q - 1.
  issue_x(0);
  issue_w(0);
  for (int q = 1; q < 5 && q < Q; ++q) issue_x(q);
  if (Q > 1) issue_w(1);
  for (int slab = 0; slab < a.nslab; ++slab) {
    for (int c = 0; c < NC; ++c) {
      const int q = slab * NC + c;
      if (q + 4 < Q)
        fr_publish<kVmcnt5>();
      else if (q + 1 < Q)
        fr_publish<kVmcnt3>();
      else
        fr_publish<kVmcnt0>();
      const int wbuf = q % kFrWBufs;
      if (c == 0) reset(wbuf);
      compute(wbuf, q % kFrXBufs, q + 5, q + 2);
    }
    fold(slab);
  }
  __syncthreads();

  // merge the 4 lists of every token (layout [list][slot][token] and
  // [list][token]: consecutive tokens on consecutive addresses)
  float2* ml = (float2*)smem;
  float2* mz = ml + kFrLists * K * kFrTokens;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int token = 64 * wt + 32 * g + col;
    const int list = 2 * we + hf;
#pragma unroll
    for (int j = 0; j < K; ++j) ml[(list * K + j) * kFrTokens + token] = make_float2(T[g][j], __int_as_float(P[g][j]));
    if (FULL) mz[list * kFrTokens + token] = make_float2(mr[g], zr[g]);
  }
  __syncthreads();
  if (tid >= kFrTokens) return;
  const long long n = tb0 + tid;
  if (n >= a.N) return;
  float V[K];
  int IX[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    V[j] = -__builtin_inff();
    IX[j] = 0x7fffffff;
  }
  for (int l = 0; l < kFrLists; ++l) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float2 e = ml[(l * K + j) * kFrTokens + tid];
      const int p = __float_as_int(e.y);
      if (p >= 0) ordered_insert<K>(V, IX, e.x, p);
    }
  }
  float lse = 0.f;
  if (FULL) {
    float mm = kLowest;
    for (int l = 0; l < kFrLists; ++l) mm = fmaxf(mm, mz[l * kFrTokens + tid].x);
    float zt = 0.f;
    for (int l = 0; l < kFrLists; ++l) {
      const float2 e = mz[l * kFrTokens + tid];
      zt += e.y * __builtin_amdgcn_exp2f((e.x - mm) * kLog2e);
    }
    lse = mm + __builtin_amdgcn_logf(zt) * kLn2;
  }
  float gw[K];
  if (FULL) {
#pragma unroll
    for (int j = 0; j < K; ++j) gw[j] = __builtin_amdgcn_exp2f((V[j] - lse) * kLog2e);
  } else {
    // Fig. 12: softmax over the k selected logits, maximum subtracted
    float denom = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      gw[j] = (j < a.k) ? __builtin_amdgcn_exp2f((V[j] - V[0]) * kLog2e) : 0.f;
      denom += gw[j];
    }
    const float inv = 1.f / denom;
#pragma unroll
    for (int j = 0; j < K; ++j) gw[j] *= inv;
  }
  const size_t o = (size_t)n * a.k;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (j < a.k) {
      a.out_idx[o + j] = IX[j];
      a.out_gate[o + j] = gw[j];
      if (a.out_logit) a.out_logit[o + j] = V[j];
    }
  }
  if (FULL && a.out_lse) a.out_lse[n] = lse;
}

hipError_t launch_fullrank_tiled(const uint16_t* X, long long N, int h, const uint16_t* W, int M,
                                 const float* bias, int k, bool full, int* out_idx, float* out_gate,
                                 float* out_logit, float* out_lse, void* ws, hipStream_t stream) {
  const int nslab = (M + kFrSlab - 1) / kFrSlab;
  uint16_t* Wq = (uint16_t*)ws;
  float* biasq = (float*)((char*)ws + (size_t)nslab * kFrSlab * h * 2);
  const long long units = (long long)nslab * (h / kFrChunk) * kFrUnitsW;
  hipLaunchKernelGGL(fr_pack_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream, W, bias, h, M,
                     nslab, Wq, biasq);
  FrTiledArgs a;
  a.X = X;
  a.Wq = Wq;
  a.biasq = biasq;
  a.out_idx = out_idx;
  a.out_gate = out_gate;
  a.out_logit = out_logit;
  a.out_lse = full ? out_lse : nullptr;
  a.N = N;
  a.h = h;
  a.nslab = nslab;
  a.k = k;
  const dim3 grid((unsigned)((N + kFrTokens - 1) / kFrTokens));
  if (full)
    hipLaunchKernelGGL(fr_tiled_kernel<true>, grid, dim3(kFrThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(fr_tiled_kernel<false>, grid, dim3(kFrThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace more
