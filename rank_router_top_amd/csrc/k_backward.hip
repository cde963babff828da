// Backward pass of the low-rank router: kernel instances and launch.
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. F.2.2 (eq. 10-12) and Algorithm 3.
#include "more_backward.h"

namespace more {

__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (bf16)x); }
__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 values -> bf16 hi + lo operands (8 each): x ~ hi + lo to ~2^-17.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16 a = (bf16)x[e];
    hi[e] = a;
    lo[e] = (bf16)(x[e] - (float)a);
  }
}

// --------------------------------------------------------------- packing
// One thread per sweep position p (0 .. Mpad-1).
__global__ __launch_bounds__(256) void bwd_pack_kernel(BwdArgs a) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  const int mpad = a.NT * kTile;
  if (p >= mpad) return;
  const int e = a.perm[p];
  const bool valid = e >= 0 && e < a.M;
  const float pb = (valid && a.pbar) ? a.pbar[e] : 0.f;
  a.pbpos[p] = pb;
  const int t = p >> 5, i = p & 31;
  a.pbq[(2 * t + ((i >> 2) & 1)) * 16 + 4 * (i >> 3) + (i & 3)] = pb;
  if (valid) {
    a.invpos[e] = p;
    for (int rho = 0; rho < kBwdRow; ++rho) a.R2t[(size_t)e * kBwdRow + rho] = rho < a.r ? a.R2[(size_t)rho * a.M + e] : 0;
  }
  // A operand of zbar^T: MFMA m of tile t, lane (rho, hf), K slot e' holds
  // row i = 16m + 8(e'/4) + 4hf + e'%4 of the tile
  const int m = i >> 4, rem = i & 15;
  const int hf = (rem >> 2) & 1, ep = 4 * (rem >> 3) + (rem & 3);
  for (int rho = 0; rho < kBwdRow; ++rho)
    a.R2b[(((size_t)t * 2 + m) * kWave + rho + 32 * hf) * 8 + ep] =
        (valid && rho < a.r) ? a.R2[(size_t)rho * a.M + e] : (uint16_t)0;
}

// ------------------------------------------------------ token-stationary
template <int R16>
__global__ __launch_bounds__(64 * kBwdTokWaves) void bwd_tok_kernel(BwdArgs a) {
  extern __shared__ __align__(16) char bt_lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NT = a.NT;
  float* lb = (float*)bt_lds;              // bias * log2 e, accumulator layout
  float* lp = lb + NT * 32;                // pbar, accumulator layout
  for (int i = threadIdx.x; i < NT * 32; i += 64 * kBwdTokWaves) {
    lb[i] = a.biasp[i] * kLog2e;
    lp[i] = a.pbq[i];
  }
  __syncthreads();
  const int hf = lane >> 5, tok = lane & 31;
  const int W = gridDim.x * kBwdTokWaves;
  const rsrc_t r2d = make_rsrc(a.R2p, NT * R16 * 1024);
  const rsrc_t r2b = make_rsrc(a.R2b, NT * 2048);
  for (long long j = (long long)blockIdx.x * kBwdTokWaves + wave; j < a.NB; j += W) {
    const long long n = j * kTile + tok;
    const bool ok = n < a.N;
    const rsrc_t zd = make_rsrc((const char*)a.Z + (size_t)j * z_block_bytes(R16), z_block_bytes(R16));
    bf16x8 zh[R16], zl[R16];
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      zh[m] = buf_load(zd, lane * 16 + m * 1024, 0);
      zl[m] = buf_load(zd, lane * 16 + (R16 + m) * 1024, 0);
    }
    // The logits come out in log2 units and already shifted by -lse: z enters
    // scaled by log2 e (hi + lo again), the bias from LDS is scaled, and one
    // more MFMA adds -lse log2 e of each token (B operand: its hi and lo in K
    // slots 0 and 1 of the token's lane; A operand: ones in those slots), so
    // P = exp2(acc) with no per-logit VALU work.  Tokens past N get -1e30.
    bf16x8 sh[R16], sl[R16];
#pragma unroll
    for (int m = 0; m < R16; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = ((float)zh[m][e] + (float)zl[m][e]) * kLog2e;
        sh[m][e] = (bf16)x;
        sl[m][e] = (bf16)(x - (float)sh[m][e]);
      }
    const float nl = ok ? -a.lse[n] * kLog2e : -1e30f;
    bf16x8 one, shift;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      one[e] = (bf16)0.f;
      shift[e] = (bf16)0.f;
    }
    if (hf == 0) {
      one[0] = (bf16)1.f;
      one[1] = (bf16)1.f;
      const bf16 nh = (bf16)nl;
      shift[0] = nh;
      shift[1] = (bf16)(nl - (float)nh);
    }
    // weight operands of tile t + 1 are requested before tile t is computed
    bf16x8 wc[R16], wn[R16];
    auto load_w = [&](int t, bf16x8 (&w)[R16]) {
#pragma unroll
      for (int m = 0; m < R16; ++m) w[m] = buf_load(r2d, lane * 16 + m * 1024, t * R16 * 1024);
    };
    auto logits = [&](int t) {
      load_w(t + 1 < NT ? t + 1 : t, wn);
      floatx16 acc = *(const floatx16*)(lb + (2 * t + hf) * 16);
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(wc[m], sh[m], acc);
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(wc[m], sl[m], acc);
      acc = mfma_bf16(one, shift, acc);
#pragma unroll
      for (int m = 0; m < R16; ++m) wc[m] = wn[m];
      return acc;
    };
    // sweep 1: g = sum over experts of pbar P (this lane's 16 rows, then both halves)
    float gp[4] = {0.f, 0.f, 0.f, 0.f};
    load_w(0, wc);
    for (int t = 0; t < NT; ++t) {
      const floatx16 acc = logits(t);
      const floatx16 pq = *(const floatx16*)(lp + (2 * t + hf) * 16);
#pragma unroll
      for (int v = 0; v < 16; ++v) gp[v & 3] += __builtin_amdgcn_exp2f(acc[v]) * pq[v];
    }
    const float gl = (gp[0] + gp[1]) + (gp[2] + gp[3]);
    const float g = gl + partner_f32(gl, hf != 0);
    if (ok && hf == 0) a.g[n] = g;
    // sweep 2: dense ybar -> zbar^T (rows rho, column = this token)
    floatx16 zb;
#pragma unroll
    for (int v = 0; v < 16; ++v) zb[v] = 0.f;
    load_w(0, wc);
    bf16x8 ac[2], an[2];
    ac[0] = buf_load(r2b, lane * 16, 0);
    ac[1] = buf_load(r2b, lane * 16, 1024);
    for (int t = 0; t < NT; ++t) {
      const int tn = t + 1 < NT ? t + 1 : t;
      an[0] = buf_load(r2b, lane * 16, tn * 2048);
      an[1] = buf_load(r2b, lane * 16, tn * 2048 + 1024);
      const floatx16 acc = logits(t);
      const floatx16 pq = *(const floatx16*)(lp + (2 * t + hf) * 16);
      float d[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) d[v] = __builtin_amdgcn_exp2f(acc[v]) * (pq[v] - g);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x8 hi, lo;
        split8(d + 8 * m, hi, lo);
        zb = mfma_bf16(ac[m], hi, zb);
        zb = mfma_bf16(ac[m], lo, zb);
      }
      ac[0] = an[0];
      ac[1] = an[1];
    }
    // sparse part: tvbar times the selected columns of R2 (rows 8q + 4hf .. +3)
    if (ok) {
      for (int c = 0; c < a.k; ++c) {
        int e = a.idx[n * a.k + c];
        e = e < 0 ? 0 : (e >= a.M ? a.M - 1 : e);
        const float w = a.tv[n * a.k + c];
        if (hf == 0) a.selpos[n * a.k + c] = a.invpos[e] * 32 + tok;
        const uint16_t* col = a.R2t + (size_t)e * kBwdRow + 4 * hf;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint2 u = *(const uint2*)(col + 8 * q);
          zb[4 * q + 0] += w * bf16_val((uint16_t)(u.x & 0xffff));
          zb[4 * q + 1] += w * bf16_val((uint16_t)(u.x >> 16));
          zb[4 * q + 2] += w * bf16_val((uint16_t)(u.y & 0xffff));
          zb[4 * q + 3] += w * bf16_val((uint16_t)(u.y >> 16));
        }
      }
      // zbar row: register 4q + e is rank 8q + 4hf + e
      float* zr = a.zbar + n * kBwdRow + 4 * hf;
#pragma unroll
      for (int q = 0; q < 4; ++q) *(float4*)(zr + 8 * q) = make_float4(zb[4 * q], zb[4 * q + 1], zb[4 * q + 2], zb[4 * q + 3]);
      // z row (fp32 = hi + lo): K slot e of step m is rank 16m + 8(e/4) + 4hf + e%4
      float* zz = a.zrm + n * kBwdRow + 4 * hf;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = m < R16 ? (float)zh[m < R16 ? m : 0][e] + (float)zl[m < R16 ? m : 0][e] : 0.f;
        *(float4*)(zz + 16 * m) = make_float4(v[0], v[1], v[2], v[3]);
        *(float4*)(zz + 16 * m + 8) = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
}

// ----------------------------------------------------- expert-stationary
// Workgroup of kBwdExpWaves waves; wave w owns TW consecutive expert tiles.
// All waves walk the same token blocks (s, s + slots, ...): the block's
// operands (z in the B layout, lse, g, z rows, the selections) are staged once
// in LDS by the whole workgroup, one block ahead (global loads issued before
// the current block is swept, written to the other LDS buffer after it).
template <int R16, int NS>
__global__ __launch_bounds__(64 * kBwdExpWaves) void bwd_exp_kernel(BwdArgs a) {
  constexpr int TW = kBwdExpTiles;
  constexpr int NTH = 64 * kBwdExpWaves;
  constexpr int ZB = 2 * R16 * 1024;              // z block bytes
  constexpr int SELMAX = 64 * NS;                 // >= 32 k entries (NS = ceil(32 k / 64))
  constexpr int ZRS = kBwdRow + 4;
  constexpr int DTS = kTile + 4;                  // padded expert-column row of the tvbar tile
  constexpr int DTT = kTile * DTS;                // floats of one tile
  struct Buf {
    u32x4 z[ZB / 16];
    float lse[kTile], g[kTile];
    float zr[kTile * ZRS];   // z rows, padded to ZRS floats (the hf halves read other banks)
    int sp[SELMAX];
    float sv[SELMAX];
  };
  __shared__ __align__(16) Buf buf[2];
  __shared__ __align__(16) float dt[kBwdExpWaves][TW * DTT];   // per wave: tvbar of its tiles [tile][expert col][token]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x / a.GE, gq = blockIdx.x % a.GE;
  const int t0 = (gq * kBwdExpWaves + wave) * TW;
  const int hf = lane >> 5, col = lane & 31;
  const int mpad = a.NT * kTile;
  float* my = dt[wave];
  const rsrc_t r2d = make_rsrc(a.R2p, a.NT * R16 * 1024);
  bf16x8 w[TW][R16];
  float pb[TW];
  // the bias of the lane's expert (log2 units) enters with one MFMA per tile:
  // B operand bias hi, lo in K slots 0 and 1, A operand ones there
  bf16x8 bo[TW], one;
#pragma unroll
  for (int e = 0; e < 8; ++e) one[e] = (bf16)((hf == 0 && e < 2) ? 1.f : 0.f);
  {
    const int bidx = ((col >> 2) & 1) * 16 + 4 * (col >> 3) + (col & 3);
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      const int t = t0 + u < a.NT ? t0 + u : a.NT - 1;
#pragma unroll
      for (int m = 0; m < R16; ++m) w[u][m] = buf_load(r2d, lane * 16 + m * 1024, t * R16 * 1024);
      const float bv = a.biasp[t * 32 + bidx];
      const float b2 = bv > -__builtin_inff() ? bv * kLog2e : -1e30f;   // padding rows: P = 0
      pb[u] = a.pbpos[t * 32 + col];
#pragma unroll
      for (int e = 0; e < 8; ++e) bo[u][e] = (bf16)0.f;
      if (hf == 0) {
        bo[u][0] = (bf16)b2;
        bo[u][1] = (bf16)(b2 - (float)bo[u][0]);
      }
    }
  }
  floatx16 r2acc[TW];
  float bacc[TW];
#pragma unroll
  for (int u = 0; u < TW; ++u) {
#pragma unroll
    for (int v = 0; v < 16; ++v) r2acc[u][v] = 0.f;
    bacc[u] = 0.f;
  }
  const long long nk = a.N * a.k;
  const int nsel = kTile * a.k;
  // staging: each thread moves a fixed share of the block's operands
  constexpr int ZCH = ZB / 16;                    // 16-byte chunks of z
  constexpr int ZRC = kTile * kBwdRow / 4;        // float4 chunks of the z rows
  struct Pre {
    u32x4 z[(ZCH + NTH - 1) / NTH], zl[(ZCH + NTH - 1) / NTH];   // hi chunk c and lo chunk c
    float4 zr[(ZRC + NTH - 1) / NTH];
    float lse, g;
    int sp[(SELMAX + NTH - 1) / NTH];
    float sv[(SELMAX + NTH - 1) / NTH];
  };
  auto fetch = [&](long long j, Pre& P) {
    const long long n0 = j * kTile;
    const u32x4* zsrc = (const u32x4*)((const char*)a.Z + (size_t)j * z_block_bytes(R16));
#pragma unroll
    for (int i = 0; i < (ZCH + NTH - 1) / NTH; ++i) {
      const int c = tid + NTH * i;
      P.z[i] = zsrc[c < ZCH / 2 ? c : 0];
      P.zl[i] = zsrc[ZCH / 2 + (c < ZCH / 2 ? c : 0)];
    }
#pragma unroll
    for (int i = 0; i < (ZRC + NTH - 1) / NTH; ++i) {
      const int c = tid + NTH * i;
      const long long row = n0 + (c < ZRC ? c : 0) / (kBwdRow / 4);
      P.zr[i] = *(const float4*)(a.zrm + (row < a.N ? row : a.N - 1) * kBwdRow + 4 * ((c < ZRC ? c : 0) % (kBwdRow / 4)));
    }
    const long long tk = n0 + (tid & 31);
    P.lse = a.lse[tk < a.N ? tk : a.N - 1];
    P.g = a.g[tk < a.N ? tk : a.N - 1];
#pragma unroll
    for (int i = 0; i < (SELMAX + NTH - 1) / NTH; ++i) {
      long long q = n0 * a.k + tid + NTH * i;
      q = q < nk ? q : nk - 1;
      P.sp[i] = a.selpos[q];
      P.sv[i] = a.tv[q];
    }
  };
  auto stage = [&](long long j, const Pre& P, Buf& B) {
    const long long n0 = j * kTile;
    // z scaled by log2 e (hi + lo again): the logits come out in log2 units
#pragma unroll
    for (int i = 0; i < (ZCH + NTH - 1) / NTH; ++i) {
      const int c = tid + NTH * i;
      if (c < ZCH / 2) {
        const bf16x8 hv = __builtin_bit_cast(bf16x8, P.z[i]);
        const bf16x8 lv = __builtin_bit_cast(bf16x8, P.zl[i]);
        bf16x8 h2, l2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = ((float)hv[e] + (float)lv[e]) * kLog2e;
          h2[e] = (bf16)x;
          l2[e] = (bf16)(x - (float)h2[e]);
        }
        B.z[c] = __builtin_bit_cast(u32x4, h2);
        B.z[ZCH / 2 + c] = __builtin_bit_cast(u32x4, l2);
      }
    }
#pragma unroll
    for (int i = 0; i < (ZRC + NTH - 1) / NTH; ++i) {
      const int c = tid + NTH * i;
      if (c < ZRC) {
        const bool ok = n0 + c / (kBwdRow / 4) < a.N;
        *(float4*)(B.zr + (c / (kBwdRow / 4)) * ZRS + 4 * (c % (kBwdRow / 4))) = ok ? P.zr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    if (tid < kTile) {
      const bool ok = n0 + tid < a.N;
      B.lse[tid] = ok ? -P.lse * kLog2e : -__builtin_inff();   // accumulator start: tokens past N give P = 0
      B.g[tid] = P.g;
    }
#pragma unroll
    for (int i = 0; i < (SELMAX + NTH - 1) / NTH; ++i) {
      const int q = tid + NTH * i;
      if (q < SELMAX) {
        const bool ok = q < nsel && n0 + q / a.k < a.N;
        B.sp[q] = ok ? P.sp[i] : -1;
        B.sv[q] = P.sv[i];
      }
    }
  };
  auto work = [&](const Buf& B) {
    bf16x8 zh[R16], zl[R16];
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      zh[m] = __builtin_bit_cast(bf16x8, B.z[m * 64 + lane]);
      zl[m] = __builtin_bit_cast(bf16x8, B.z[(R16 + m) * 64 + lane]);
    }
    floatx16 c0;
    float gv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 l4 = *(const float4*)(B.lse + 8 * q + 4 * hf);
      const float4 g4 = *(const float4*)(B.g + 8 * q + 4 * hf);
      c0[4 * q] = l4.x; c0[4 * q + 1] = l4.y; c0[4 * q + 2] = l4.z; c0[4 * q + 3] = l4.w;
      gv[4 * q] = g4.x; gv[4 * q + 1] = g4.y; gv[4 * q + 2] = g4.z; gv[4 * q + 3] = g4.w;
    }
    // z^T operand: K slot e' of step m = token 16m + 8(e'/4) + 4hf + e'%4, rank = col
    bf16x8 zth[2], ztl[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = B.zr[(16 * m + 8 * (e >> 2) + 4 * hf + (e & 3)) * ZRS + col];
      split8(x, zth[m], ztl[m]);
    }
    int spos[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) spos[i] = B.sp[lane + 64 * i];
    // The TW tiles are processed phase by phase (logits, P and ybar, selected
    // entries, MFMAs), so the dependent chains of different tiles interleave.
    floatx16 acc[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) acc[u] = c0;
#pragma unroll
    for (int m = 0; m < R16; ++m)
#pragma unroll
      for (int u = 0; u < TW; ++u) acc[u] = mfma_bf16(zh[m], w[u][m], acc[u]);
#pragma unroll
    for (int m = 0; m < R16; ++m)
#pragma unroll
      for (int u = 0; u < TW; ++u) acc[u] = mfma_bf16(zl[m], w[u][m], acc[u]);
#pragma unroll
    for (int u = 0; u < TW; ++u) acc[u] = mfma_bf16(one, bo[u], acc[u]);
    float d[TW][16];
#pragma unroll
    for (int u = 0; u < TW; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) d[u][v] = __builtin_amdgcn_exp2f(acc[u][v]) * (pb[u] - gv[v]);
    // the block's tvbar in the wave's tiles, dense in LDS: cleared, scattered
    // (a token selects an expert at most once), then read like ybar itself
#pragma unroll
    for (int i = 0; i < TW * DTT / 4 / 64; ++i)
      *(float4*)(my + 4 * (lane + 64 * i)) = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int tl = (spos[i] >> 10) - t0;
      if (spos[i] >= 0 && tl >= 0 && tl < TW) my[tl * DTT + ((spos[i] >> 5) & 31) * DTS + (spos[i] & 31)] = B.sv[lane + 64 * i];
    }
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      const float* row = my + u * DTT + col * DTS + 4 * hf;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 x = *(const float4*)(row + 8 * q);
        d[u][4 * q] += x.x;
        d[u][4 * q + 1] += x.y;
        d[u][4 * q + 2] += x.z;
        d[u][4 * q + 3] += x.w;
      }
    }
    bf16x8 dh[TW][2], dl[TW][2];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      float bs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) bs += d[u][v];
      bacc[u] += bs;
#pragma unroll
      for (int m = 0; m < 2; ++m) split8(d[u] + 8 * m, dh[u][m], dl[u][m]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int u = 0; u < TW; ++u) {
        r2acc[u] = mfma_bf16(zth[m], dh[u][m], r2acc[u]);
        r2acc[u] = mfma_bf16(zth[m], dl[u][m], r2acc[u]);
        r2acc[u] = mfma_bf16(ztl[m], dh[u][m], r2acc[u]);
      }
  };
  Pre P;
  long long j = s;
  fetch(j, P);
  stage(j, P, buf[0]);
  __syncthreads();
  int cur = 0;
  for (; j < a.NB; j += a.slotsE) {
    const bool more = j + a.slotsE < a.NB;
    if (more) fetch(j + a.slotsE, P);
    work(buf[cur]);
    if (more) stage(j + a.slotsE, P, buf[cur ^ 1]);
    __syncthreads();   // next buffer complete; the current one is free again
    cur ^= 1;
  }
  // partials: R2bar^T rows rho = 8(v/4) + 4hf + v%4, column = this lane's position
#pragma unroll
  for (int u = 0; u < TW; ++u) {
    const int t = t0 + u;
    if (t >= a.NT) continue;
    const int p = t * kTile + col;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rho = 8 * (v >> 2) + 4 * hf + (v & 3);
      a.r2part[((size_t)s * kBwdRow + rho) * mpad + p] = r2acc[u][v];
    }
    const float tot = bacc[u] + partner_f32(bacc[u], hf != 0);
    if (hf == 0) a.bpart[(size_t)s * mpad + p] = tot;
  }
}

// ------------------------------------------------------------ X stream
// Each wave owns HT h tiles (32 columns each) and walks the token blocks of
// its slot, one block of loads ahead.  X rows arrive with 16-byte loads and
// go into the wave's LDS area transposed ([column][token]), so the B operand
// of R1bar^T += zbar^T X (K = the block's tokens) is one 16-byte LDS read.
// xbar^T = R1 zbar^T leaves four consecutive columns of one token per lane
// and register group; they are staged in LDS by token rows and leave with
// 16-byte stores.
template <int R16>
__global__ __launch_bounds__(64 * kBwdXWaves) void bwd_x_kernel(BwdArgs a) {
  constexpr int HT = kBwdXTiles;
  constexpr int WC = HT * kTile;                 // columns of one wave
  constexpr int NCH = kTile * WC / 8 / 64;       // 16-byte chunks of a block slice per lane
  // padded rows: a column of X^T is 32 tokens + 8 (80 bytes), so the 16-byte
  // reads of 16 consecutive columns and the transposed 2-byte writes spread
  // over the banks; a token row of xbar is WC columns + 8 (16-byte aligned)
  constexpr int XS = kTile + 8, YS = WC + 8;
  __shared__ __align__(16) uint16_t xs_all[kBwdXWaves][WC * XS];   // X^T [column][token]
  __shared__ __align__(16) uint16_t ys_all[kBwdXWaves][kTile * YS];   // xbar [token][column]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = blockIdx.x / a.GX, gq = blockIdx.x % a.GX;
  const int ht0 = (gq * kBwdXWaves + wave) * HT;
  const int nht = a.h / kTile;
  if (ht0 >= nht) return;
  const int c0 = ht0 * kTile;
  const int ncol = (nht - ht0 < HT ? nht - ht0 : HT) * kTile;
  uint32_t* xs32 = (uint32_t*)xs_all[wave];
  // word of token pair p (tokens 2p, 2p + 1) in column c: the 16-byte groups
  // of 4 pairs are swizzled by bits 3-4 of the column, so the transposed
  // writes of 8 columns x 4 pairs spread over the banks while a group of 8
  // consecutive tokens stays one 16-byte read
  auto xs_word = [](int c, int p) { return c * (XS / 2) + 4 * ((p >> 2) ^ ((c >> 3) & 3)) + (p & 3); };
  uint16_t* ys = ys_all[wave];
  const int hf = lane >> 5, col = lane & 31;
  // R1 rows as the A operand of xbar^T: lane (column, hf), K slot e' = rank 16m + 8hf + e'
  bf16x8 br[HT][R16];
#pragma unroll
  for (int u = 0; u < HT; ++u) {
    const int hc = c0 + (u * kTile < ncol ? u * kTile : 0) + col;
#pragma unroll
    for (int m = 0; m < R16; ++m)
      br[u][m] = __builtin_bit_cast(bf16x8, *(const u32x4*)(a.R1 + (size_t)hc * a.r + 16 * m + 8 * hf));
  }
  floatx16 r1acc[HT];
#pragma unroll
  for (int u = 0; u < HT; ++u)
#pragma unroll
    for (int v = 0; v < 16; ++v) r1acc[u][v] = 0.f;
  // loads of one block: X slice chunks (token q / (WC/8), 8 columns) and zbar
  struct Blk {
    u32x4 x[NCH];
    float4 za[2 * R16];   // zbar row of token `col`, ranks 16m + 8hf .. +7
    float zt[16];         // zbar[token 16m + 8hf + e][rank col]
  };
  auto load_blk = [&](long long j, Blk& B) {
    const long long n0 = j * kTile;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = lane + 64 * i;
      const long long row = n0 + q / (WC / 8);
      const int cc = (q % (WC / 8)) * 8;
      const long long rr = row < a.N ? row : a.N - 1;
      const int c = cc < ncol ? cc : 0;
      B.x[i] = *(const u32x4*)(a.X + rr * a.h + c0 + c);   // rows / columns past the end: masked at use
    }
    const long long tk = n0 + col < a.N ? n0 + col : a.N - 1;
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      B.za[2 * m] = *(const float4*)(a.zbar + tk * kBwdRow + 16 * m + 8 * hf);
      B.za[2 * m + 1] = *(const float4*)(a.zbar + tk * kBwdRow + 16 * m + 8 * hf + 4);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const long long tt = n0 + 16 * (e >> 3) + 8 * hf + (e & 7);
      B.zt[e] = a.zbar[(tt < a.N ? tt : a.N - 1) * kBwdRow + col];
    }
  };
  auto work = [&](long long j, const Blk& B) {
    __builtin_amdgcn_sched_barrier(0);
    const long long n0 = j * kTile;
    // X slice -> LDS, transposed; rows past N and columns past the wave's end
    // are zero.  Lanes l and l ^ 8 hold tokens 2p and 2p + 1 of the same 8
    // columns: they swap half their columns (DPP row_ror:8), and each writes
    // 4 words holding both tokens of one column.
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = lane + 64 * i;
      const int tok = q / (WC / 8);
      const int cc = (q % (WC / 8)) * 8;
      const bool ok = n0 + tok < a.N && cc < ncol;
      const u32x4 v = ok ? B.x[i] : u32x4{0u, 0u, 0u, 0u};
      const bool odd = (tok & 1) != 0;   // = (lane & 8) != 0
      const uint32_t keep0 = odd ? v[2] : v[0], keep1 = odd ? v[3] : v[1];
      const uint32_t send0 = odd ? v[0] : v[2], send1 = odd ? v[1] : v[3];
      const uint32_t recv0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send0, 0x128, 0xf, 0xf, false);
      const uint32_t recv1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send1, 0x128, 0xf, 0xf, false);
      const uint32_t ev0 = odd ? recv0 : keep0, od0 = odd ? keep0 : recv0;   // even / odd token, 2 columns
      const uint32_t ev1 = odd ? recv1 : keep1, od1 = odd ? keep1 : recv1;
      const uint32_t w4[4] = {(ev0 & 0xffffu) | (od0 << 16), (ev0 >> 16) | (od0 & 0xffff0000u),
                              (ev1 & 0xffffu) | (od1 << 16), (ev1 >> 16) | (od1 & 0xffff0000u)};
      const int c0 = cc + (odd ? 4 : 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) xs32[xs_word(c0 + e, tok >> 1)] = w4[e];
    }
    const bool tok_ok = n0 + col < a.N;
    bf16x8 zbh[R16], zbl[R16], zth[2], ztl[2];
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      float x[8];
      const float4 p0 = B.za[2 * m], p1 = B.za[2 * m + 1];
      x[0] = p0.x; x[1] = p0.y; x[2] = p0.z; x[3] = p0.w; x[4] = p1.x; x[5] = p1.y; x[6] = p1.z; x[7] = p1.w;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = tok_ok ? x[e] : 0.f;
      split8(x, zbh[m], zbl[m]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = n0 + 16 * m + 8 * hf + e < a.N ? B.zt[8 * m + e] : 0.f;
      split8(y, zth[m], ztl[m]);
    }
#pragma unroll
    for (int u = 0; u < HT; ++u) {
      if (u * kTile >= ncol) break;
      // xbar^T tile: rows = columns u*32 + 8(v/4) + 4hf + v%4, column = token
      floatx16 xa;
#pragma unroll
      for (int v = 0; v < 16; ++v) xa[v] = 0.f;
#pragma unroll
      for (int m = 0; m < R16; ++m) {
        xa = mfma_bf16(br[u][m], zbh[m], xa);
        xa = mfma_bf16(br[u][m], zbl[m], xa);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (uint32_t)bf16_bits(xa[4 * q]) | ((uint32_t)bf16_bits(xa[4 * q + 1]) << 16);
        const uint32_t hi = (uint32_t)bf16_bits(xa[4 * q + 2]) | ((uint32_t)bf16_bits(xa[4 * q + 3]) << 16);
        *(uint2*)(ys + col * YS + u * kTile + 8 * q + 4 * hf) = make_uint2(lo, hi);
      }
      // R1bar^T partial: rows = ranks, column = h; K = the block's tokens
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 xb = __builtin_bit_cast(bf16x8, *(const u32x4*)(xs32 + xs_word(u * kTile + col, 8 * m + 4 * hf)));
        r1acc[u] = mfma_bf16(zth[m], xb, r1acc[u]);
        r1acc[u] = mfma_bf16(ztl[m], xb, r1acc[u]);
      }
    }
    // xbar rows of the block: 16-byte chunks
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = lane + 64 * i;
      const int tok = q / (WC / 8);
      const int cc = (q % (WC / 8)) * 8;
      const u32x4 v = *(const u32x4*)(ys + tok * YS + cc);
      if (n0 + tok < a.N && cc < ncol) *(u32x4*)(a.xbar + (n0 + tok) * a.h + c0 + cc) = v;
    }
  };
  Blk b0, b1;
  const long long st = a.slotsX, last = a.NB - 1;
  long long j = s;
  load_blk(j, b0);
  for (;; j += 2 * st) {
    load_blk(j + st < last ? j + st : last, b1);
    work(j, b0);
    if (j + st >= a.NB) break;
    load_blk(j + 2 * st < last ? j + 2 * st : last, b0);
    work(j + st, b1);
    if (j + 2 * st >= a.NB) break;
  }
  // partial rows [slot][h][32]: rank 8(v/4) + 4hf + v%4 of column h
#pragma unroll
  for (int u = 0; u < HT; ++u) {
    if (u * kTile >= ncol) break;
    const int hc = c0 + u * kTile + col;
    float* dst = a.r1part + ((size_t)s * a.h + hc) * kBwdRow + 4 * hf;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(float4*)(dst + 8 * q) = make_float4(r1acc[u][4 * q], r1acc[u][4 * q + 1], r1acc[u][4 * q + 2], r1acc[u][4 * q + 3]);
  }
}

// ------------------------------------------------------------- reduce
// One thread per output element, slots summed in order.  Elements:
// [0, r*Mpad): R2bar (rank, position); [r*Mpad, r*Mpad + Mpad): bbar by
// position; then h*r elements of R1bar.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long mpad = (long long)a.NT * kTile;
  const long long n2 = (long long)a.r * mpad, nb = mpad, n1 = (long long)a.h * a.r;
  if (i < n2) {
    const int rho = (int)(i / mpad), p = (int)(i % mpad);
    float s = 0.f;
    for (int q = 0; q < a.slotsE; ++q) s += a.r2part[((size_t)q * kBwdRow + rho) * mpad + p];
    const int e = a.perm[p];
    if (e >= 0 && e < a.M) a.r2grad[(size_t)rho * a.M + e] = s;
  } else if (i < n2 + nb) {
    const int p = (int)(i - n2);
    float s = 0.f;
    for (int q = 0; q < a.slotsE; ++q) s += a.bpart[(size_t)q * mpad + p];
    const int e = a.perm[p];
    if (a.bgrad && e >= 0 && e < a.M) a.bgrad[e] = s;
  } else if (i < n2 + nb + n1) {
    const long long q0 = i - n2 - nb;
    const int hc = (int)(q0 / a.r), rho = (int)(q0 % a.r);
    float s = 0.f;
    for (int q = 0; q < a.slotsX; ++q) s += a.r1part[((size_t)q * a.h + hc) * kBwdRow + rho];
    a.r1grad[(size_t)hc * a.r + rho] = s;
  }
}

template <int R16>
static hipError_t launch_r(const BwdArgs& a, size_t tok_lds, int cus, hipStream_t stream) {
  const int mpad = a.NT * kTile;
  hipLaunchKernelGGL(bwd_pack_kernel, dim3((unsigned)((mpad + 255) / 256)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = hipFuncSetAttribute((const void*)bwd_tok_kernel<R16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)tok_lds)) != hipSuccess)
    return e;
  const long long tg = std::max<long long>(1, std::min<long long>(cus, ((long long)a.NB + kBwdTokWaves - 1) / kBwdTokWaves));
  hipLaunchKernelGGL(bwd_tok_kernel<R16>, dim3((unsigned)tg), dim3(64 * kBwdTokWaves), tok_lds, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.k <= 8)
    hipLaunchKernelGGL((bwd_exp_kernel<R16, 4>), dim3((unsigned)(a.slotsE * a.GE)), dim3(64 * kBwdExpWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_exp_kernel<R16, 16>), dim3((unsigned)(a.slotsE * a.GE)), dim3(64 * kBwdExpWaves), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_x_kernel<R16>, dim3((unsigned)(a.slotsX * a.GX)), dim3(64 * kBwdXWaves), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long long tot = (long long)a.r * mpad + mpad + (long long)a.h * a.r;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_backward(int r16, const BwdArgs& a, size_t tok_lds, int cus, hipStream_t stream) {
  return r16 == 1 ? launch_r<1>(a, tok_lds, cus, stream) : launch_r<2>(a, tok_lds, cus, stream);
}

}  // namespace more
