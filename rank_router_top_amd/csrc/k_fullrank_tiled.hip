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
constexpr int kFrBuf = kFrXBytes + kFrWBytes + kFrBBytes;  // one LDS buffer
constexpr int kFrUnitsW = kFrWBytes / 16;                  // 16-byte units of a weight chunk
constexpr int kFrLists = 2 * (kFrWaves / 2);               // lists per token: 4 expert quarters x 2 halves
static_assert(kFrThreads == kFrTokens * kFrChunk * 2 / 16, "one 16-byte X unit per thread");
static_assert(kFrUnitsW % kFrThreads == 0, "whole weight units per thread");
static_assert(kFrSlab == kFrThreads, "one bias value per thread");
static_assert(kFrTokens * kFrLists * (kFrKmax + 1) * 8 <= 2 * kFrBuf, "merge area fits the operand buffers");
}  // namespace

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
    const int lane = (int)(u % 64), s = (int)((u / 64) % 2), t = (int)((u / 128) % 16);
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
    const int v = (int)(u % 16), hf = (int)((u / 16) % 2), t = (int)((u / 32) % 16);
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
  __shared__ __align__(16) char smem[2 * kFrBuf];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = w & 1, we = w >> 1;
  const bool hi = lane >= 32;
  const int hf = hi ? 1 : 0, col = lane & 31;
  const long long tb0 = (long long)blockIdx.x * kFrTokens;
  const int NC = a.h / kFrChunk;   // even: h is a multiple of 2 kFrChunk
  const int Q = a.nslab * NC;

  // staging: thread tid moves 16 bytes of token xt's 64-byte chunk row (part
  // xq = K-step xq / 2, half xq % 2) and 64 bytes of the weight chunk
  const int xt = tid >> 2, xq = tid & 3;
  const long long xrow = tb0 + xt;
  const bool xok = xrow < a.N;
  const uint16_t* xsrc = a.X + (xok ? xrow : a.N - 1) * (long long)a.h + 8 * xq;
  const int xdst = (((xt >> 5) * 2 + (xq >> 1)) * kWave + (xt & 31) + 32 * (xq & 1)) * 16;

  struct Ld {
    u32x4 x;
    u32x4 w[kFrUnitsW / kFrThreads];
    float b;
  };
  auto fetch = [&](int q, Ld& L) {
    const int slab = q / NC, c = q - slab * NC;
    L.x = *(const u32x4*)(xsrc + (long long)c * kFrChunk);
    const u32x4* ws = (const u32x4*)a.Wq + (long long)q * kFrUnitsW + tid;
#pragma unroll
    for (int i = 0; i < kFrUnitsW / kFrThreads; ++i) L.w[i] = ws[i * kFrThreads];
    L.b = a.biasq[(long long)slab * kFrSlab + tid];
  };
  auto stage = [&](const Ld& L, int buf) {
    char* base = smem + buf * kFrBuf;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    *(u32x4*)(base + xdst) = xok ? L.x : zero;
    u32x4* wd = (u32x4*)(base + kFrXBytes) + tid;
#pragma unroll
    for (int i = 0; i < kFrUnitsW / kFrThreads; ++i) wd[i * kFrThreads] = L.w[i];
    ((float*)(base + kFrXBytes + kFrWBytes))[tid] = L.b;
  };

  floatx16 acc[2][4];
  auto reset = [&](int buf) {
    const float* bs = (const float*)(smem + buf * kFrBuf + kFrXBytes + kFrWBytes);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const floatx16 bv = *(const floatx16*)(bs + ((4 * we + t) * 2 + hf) * 16);
      acc[0][t] = bv;
      acc[1][t] = bv;
    }
  };
  auto compute = [&](int buf) {
    const bf16x8* xs = (const bf16x8*)(smem + buf * kFrBuf);
    const bf16x8* ws = (const bf16x8*)(smem + buf * kFrBuf + kFrXBytes);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 b0 = xs[((2 * wt + 0) * 2 + s) * kWave + lane];
      const bf16x8 b1 = xs[((2 * wt + 1) * 2 + s) * kWave + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8 av = ws[((4 * we + t) * 2 + s) * kWave + lane];
        acc[0][t] = mfma_bf16(av, b0, acc[0][t]);
        acc[1][t] = mfma_bf16(av, b1, acc[1][t]);
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
  // two LDS buffers; the loads of a chunk are issued two chunks before it is
  // staged.  A slab has an even number of chunks, so it starts in buffer 0,
  // which then also holds its bias.
  Ld L0, L1;
  fetch(0, L0);
  fetch(1, L1);
  stage(L0, 0);
  __syncthreads();
  for (int slab = 0; slab < a.nslab; ++slab) {
    reset(0);
    for (int c = 0; c < NC; c += 2) {
      const int q = slab * NC + c;
      if (q + 2 < Q) fetch(q + 2, L0);
      compute(0);
      stage(L1, 1);
      __syncthreads();
      if (q + 3 < Q) fetch(q + 3, L1);
      compute(1);
      if (q + 2 < Q) stage(L0, 0);
      __syncthreads();
    }
    fold(slab);
  }

  // merge the 8 lists of every token (layout [list][slot][token] and
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
