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
  float* lb = (float*)bt_lds;              // bias, accumulator layout
  float* lp = lb + NT * 32;                // pbar, accumulator layout
  for (int i = threadIdx.x; i < NT * 32; i += 64 * kBwdTokWaves) {
    lb[i] = a.biasp[i];
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
    const float nl = ok ? -a.lse[n] * kLog2e : -__builtin_inff();
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
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(wc[m], zh[m], acc);
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(wc[m], zl[m], acc);
#pragma unroll
      for (int m = 0; m < R16; ++m) wc[m] = wn[m];
      return acc;
    };
    // sweep 1: g = sum over experts of pbar P (this lane's 16 rows, then both halves)
    float gl = 0.f;
    load_w(0, wc);
    for (int t = 0; t < NT; ++t) {
      const floatx16 acc = logits(t);
      const floatx16 pq = *(const floatx16*)(lp + (2 * t + hf) * 16);
#pragma unroll
      for (int v = 0; v < 16; ++v) gl += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], kLog2e, nl)) * pq[v];
    }
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
      for (int v = 0; v < 16; ++v) d[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], kLog2e, nl)) * (pq[v] - g);
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
template <int R16>
__global__ __launch_bounds__(64 * kBwdExpWaves) void bwd_exp_kernel(BwdArgs a) {
  constexpr int TW = kBwdExpTiles;
  __shared__ __align__(16) float dt[kBwdExpWaves][kTile * kTile];   // per wave: ybar tile [expert col][token]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = blockIdx.x / a.GE, gq = blockIdx.x % a.GE;
  const int t0 = (gq * kBwdExpWaves + wave) * TW;
  const int hf = lane >> 5, col = lane & 31;
  const int mpad = a.NT * kTile;
  float* my = dt[wave];
  const rsrc_t r2d = make_rsrc(a.R2p, a.NT * R16 * 1024);
  bf16x8 w[TW][R16];
  float bl[TW], pb[TW];
  {
    const int bidx = ((col >> 2) & 1) * 16 + 4 * (col >> 3) + (col & 3);
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      const int t = t0 + u < a.NT ? t0 + u : a.NT - 1;
#pragma unroll
      for (int m = 0; m < R16; ++m) w[u][m] = buf_load(r2d, lane * 16 + m * 1024, t * R16 * 1024);
      bl[u] = a.biasp[t * 32 + bidx] * kLog2e;
      pb[u] = a.pbpos[t * 32 + col];
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
  const int nsel = (kTile * a.k + 63) / 64;   // selections of a block per lane (k <= 32: <= 16)
  for (long long j = s; j < a.NB; j += a.slotsE) {
    __builtin_amdgcn_sched_barrier(0);
    const long long n0 = j * kTile;
    const rsrc_t zd = make_rsrc((const char*)a.Z + (size_t)j * z_block_bytes(R16), z_block_bytes(R16));
    bf16x8 zh[R16], zl[R16];
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      zh[m] = buf_load(zd, lane * 16 + m * 1024, 0);
      zl[m] = buf_load(zd, lane * 16 + (R16 + m) * 1024, 0);
    }
    // token of register v: 8(v/4) + 4hf + v%4; lse start (-inf past N) and g
    floatx16 c0;
    float gv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const long long tk = n0 + 8 * (v >> 2) + 4 * hf + (v & 3);
      const long long tc = tk < a.N ? tk : a.N - 1;
      const float ls = a.lse[tc], gg = a.g[tc];
      c0[v] = tk < a.N ? -ls : -__builtin_inff();
      gv[v] = gg;
    }
    // z^T operand of MFMA m: lane (rho, hf), K slot e' = token 16m + 8(e'/4) + 4hf + e'%4
    bf16x8 zth[2], ztl[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const long long tk = n0 + 16 * m + 8 * (e >> 2) + 4 * hf + (e & 3);
        x[e] = tk < a.N ? a.zrm[tk * kBwdRow + col] : 0.f;
      }
      split8(x, zth[m], ztl[m]);
    }
    // the block's selections: lane takes entries lane, lane + 64, ... of the
    // 32 k (token, slot) pairs; position, and token within the block
    int spos[16];
    float sval[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      spos[i] = -1;
      sval[i] = 0.f;
      if (i < nsel) {
        const int q = lane + 64 * i;
        const long long tk = n0 + q / a.k;
        if (q < kTile * a.k && tk < a.N) {
          int ex = a.idx[n0 * a.k + q];
          ex = ex < 0 ? 0 : (ex >= a.M ? a.M - 1 : ex);   // out-of-range indices: no access outside the table
          spos[i] = a.invpos[ex] * 32 + q / a.k;            // position * 32 + token
          sval[i] = a.tv[n0 * a.k + q];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      const int t = t0 + u;
      floatx16 acc = c0;
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(zh[m], w[u][m], acc);
#pragma unroll
      for (int m = 0; m < R16; ++m) acc = mfma_bf16(zl[m], w[u][m], acc);
      float d[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) d[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], kLog2e, bl[u])) * (pb[u] - gv[v]);
      // selected (token, expert) pairs in this tile: add tvbar through the LDS tile
      bool hit = false;
#pragma unroll
      for (int i = 0; i < 16; ++i) hit = hit || (i < nsel && (spos[i] >> 10) == t);
      if (any_lane(hit)) {
        float* row = my + col * kTile + 4 * hf;
#pragma unroll
        for (int q = 0; q < 4; ++q) *(float4*)(row + 8 * q) = make_float4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i < nsel && (spos[i] >> 10) == t) my[((spos[i] >> 5) & 31) * kTile + (spos[i] & 31)] += sval[i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 x = *(const float4*)(row + 8 * q);
          d[4 * q] = x.x;
          d[4 * q + 1] = x.y;
          d[4 * q + 2] = x.z;
          d[4 * q + 3] = x.w;
        }
      }
      float bs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) bs += d[v];
      bacc[u] += bs;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x8 hi, lo;
        split8(d + 8 * m, hi, lo);
        r2acc[u] = mfma_bf16(zth[m], hi, r2acc[u]);
        r2acc[u] = mfma_bf16(zth[m], lo, r2acc[u]);
        r2acc[u] = mfma_bf16(ztl[m], hi, r2acc[u]);
      }
    }
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
template <int R16>
__global__ __launch_bounds__(64 * kBwdXWaves) void bwd_x_kernel(BwdArgs a) {
  constexpr int HT = kBwdXTiles;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = blockIdx.x / a.GX, gq = blockIdx.x % a.GX;
  const int ht0 = (gq * kBwdXWaves + wave) * HT;   // first h tile of this wave
  const int nht = a.h / kTile;
  if (ht0 >= nht) return;
  const int hf = lane >> 5, col = lane & 31;
  // R1^T operand of h tile u: lane (h column, hf), K slot e' = rank 16m + 8hf + e'
  bf16x8 br[HT][R16];
#pragma unroll
  for (int u = 0; u < HT; ++u) {
    const int hc = (ht0 + u < nht ? ht0 + u : nht - 1) * kTile + col;
#pragma unroll
    for (int m = 0; m < R16; ++m) br[u][m] = __builtin_bit_cast(bf16x8, *(const u32x4*)(a.R1 + (size_t)hc * a.r + 16 * m + 8 * hf));
  }
  floatx16 r1acc[HT];
#pragma unroll
  for (int u = 0; u < HT; ++u)
#pragma unroll
    for (int v = 0; v < 16; ++v) r1acc[u][v] = 0.f;
  for (long long j = s; j < a.NB; j += a.slotsX) {
    const long long n0 = j * kTile;
    // zbar as the A operand of xbar (lane = token, K slot = rank 16m + 8hf + e')
    // and of R1bar^T (lane = rank, K slot = token 16m + 8hf + e')
    bf16x8 zah[R16], zal[R16], zth[2], ztl[2];
#pragma unroll
    for (int m = 0; m < R16; ++m) {
      float x[8];
      const long long tk = n0 + col;
      const float* zr = a.zbar + (tk < a.N ? tk : a.N - 1) * kBwdRow + 16 * m + 8 * hf;
      const float4 p0 = *(const float4*)zr, p1 = *(const float4*)(zr + 4);
      const bool ok = tk < a.N;
      x[0] = ok ? p0.x : 0.f; x[1] = ok ? p0.y : 0.f; x[2] = ok ? p0.z : 0.f; x[3] = ok ? p0.w : 0.f;
      x[4] = ok ? p1.x : 0.f; x[5] = ok ? p1.y : 0.f; x[6] = ok ? p1.z : 0.f; x[7] = ok ? p1.w : 0.f;
      split8(x, zah[m], zal[m]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {   // the 32 tokens of the block: two K steps
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const long long tt = n0 + 16 * m + 8 * hf + e;
        y[e] = tt < a.N ? a.zbar[tt * kBwdRow + col] : 0.f;
      }
      split8(y, zth[m], ztl[m]);
    }
#pragma unroll
    for (int u = 0; u < HT; ++u) {
      if (ht0 + u >= nht) break;
      const int hc = (ht0 + u) * kTile + col;
      // xbar tile: rows = tokens 8(v/4) + 4hf + v%4, column = h
      floatx16 xa;
#pragma unroll
      for (int v = 0; v < 16; ++v) xa[v] = 0.f;
#pragma unroll
      for (int m = 0; m < R16; ++m) {
        xa = mfma_bf16(zah[m], br[u][m], xa);
        xa = mfma_bf16(zal[m], br[u][m], xa);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const long long tk = n0 + 8 * (v >> 2) + 4 * hf + (v & 3);
        if (tk < a.N) a.xbar[tk * a.h + hc] = bf16_bits(xa[v]);
      }
      // R1bar^T partial: rows = ranks, column = h; K = the block's tokens
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x8 xb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const long long tt = n0 + 16 * m + 8 * hf + e;
          const uint16_t bits = a.X[(tt < a.N ? tt : a.N - 1) * a.h + hc];
          xb[e] = tt < a.N ? __builtin_bit_cast(bf16, bits) : (bf16)0.f;
        }
        r1acc[u] = mfma_bf16(zth[m], xb, r1acc[u]);
        r1acc[u] = mfma_bf16(ztl[m], xb, r1acc[u]);
      }
    }
  }
  // partial rows [slot][h][32]: rank 8(v/4) + 4hf + v%4 of column h
#pragma unroll
  for (int u = 0; u < HT; ++u) {
    if (ht0 + u >= nht) break;
    const int hc = (ht0 + u) * kTile + col;
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
  hipLaunchKernelGGL(bwd_exp_kernel<R16>, dim3((unsigned)(a.slotsE * a.GE)), dim3(64 * kBwdExpWaves), 0, stream, a);
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
