// Expert dispatch sort + count: kernels and launch.
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. E, Fig. 9 (sort + count after the router).
#include "more_sort.h"

namespace more {

// Entry range of workgroup bid: with B a multiple of 8, XCD x (the
// workgroups bid = x mod 8) owns the contiguous blocks x B/8 .. (x+1) B/8 - 1.
__device__ __forceinline__ int sort_chunk(int bid, int B) {
  return (B & 7) == 0 ? (bid & 7) * (B >> 3) + (bid >> 3) : bid;
}

// Digit of a key in this pass; keys outside [0, M) are clamped into the
// last bin (their order is unspecified, every access stays in bounds).
__device__ __forceinline__ int sort_digit(int key, const SortPassArgs& a) {
  const unsigned u = ((unsigned)key >> a.shift) & a.mask;
  return u < (unsigned)a.bins ? (int)u : a.bins - 1;
}

// Inclusive scans over the 64 lanes of a wave with DPP row shifts and row
// broadcasts (no LDS round trip): lanes outside a step's source keep the
// identity.
__device__ __forceinline__ int wave_scan_add(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return x;
}
__device__ __forceinline__ int wave_scan_max(int x) {   // values >= -1
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x111, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x112, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x114, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x118, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x142, 0xa, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x143, 0xc, 0xf, false));
  return x;
}

// Per-block digit counts.
__global__ __launch_bounds__(kSortCountThreads) void sort_count_kernel(SortPassArgs a) {
  __shared__ int h[kSortBinsMax];
  for (int i = threadIdx.x; i < a.bins; i += kSortCountThreads) h[i] = 0;
  const int c = sort_chunk(blockIdx.x, a.B);
  const long long base = (long long)c * kSortBlock;
  const int nv = a.n - base < kSortBlock ? (int)(a.n - base) : kSortBlock;
  const int* src = a.keys_in + base;
  constexpr int V = kSortBlock / kSortCountThreads / 4;
  int4 kv[V];
  if (nv == kSortBlock) {
#pragma unroll
    for (int q = 0; q < V; ++q) kv[q] = ((const int4*)src)[q * kSortCountThreads + threadIdx.x];
  } else {
#pragma unroll
    for (int q = 0; q < V; ++q) {
      const int e = 4 * (q * kSortCountThreads + threadIdx.x);
      kv[q].x = e < nv ? src[e] : 0;
      kv[q].y = e + 1 < nv ? src[e + 1] : 0;
      kv[q].z = e + 2 < nv ? src[e + 2] : 0;
      kv[q].w = e + 3 < nv ? src[e + 3] : 0;
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < V; ++q) {
    const int e = 4 * (q * kSortCountThreads + threadIdx.x);
    if (e < nv) atomicAdd(&h[sort_digit(kv[q].x, a)], 1);
    if (e + 1 < nv) atomicAdd(&h[sort_digit(kv[q].y, a)], 1);
    if (e + 2 < nv) atomicAdd(&h[sort_digit(kv[q].z, a)], 1);
    if (e + 3 < nv) atomicAdd(&h[sort_digit(kv[q].w, a)], 1);
  }
  __syncthreads();
  int* row = a.hist + (size_t)c * a.bins;
  for (int i = threadIdx.x; i < a.bins; i += kSortCountThreads) row[i] = h[i];
}

// Workgroup g: digits 64 g .. 64 g + 63, one per lane; each of the 16 waves
// sums 16 consecutive blocks of a 256-block window (a wave's load reads 256
// contiguous bytes of one block's row), the waves' sums are combined in LDS,
// and the exclusive prefix over the blocks replaces the counts.  The last
// carry is the digit's total.
__global__ __launch_bounds__(kSortColWaves * 64) void sort_colscan_kernel(int* hist, int* tot, int B, int bins) {
  constexpr int kPer = 16;
  __shared__ int part[kSortColWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d = blockIdx.x * 64 + lane;
  const bool dok = d < bins;
  int carry = 0;
  for (int c0 = 0; c0 < B; c0 += kSortColWaves * kPer) {
    const int b0 = c0 + w * kPer;
    int v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = (dok && b0 + i < B) ? hist[(size_t)(b0 + i) * bins + d] : 0;
    int s = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) s += v[i];
    part[w][lane] = s;
    __syncthreads();
    int before = carry, total = carry;
#pragma unroll
    for (int k = 0; k < kSortColWaves; ++k) {
      const int p = part[k][lane];
      before += k < w ? p : 0;
      total += p;
    }
    int run = before;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (dok && b0 + i < B) hist[(size_t)(b0 + i) * bins + d] = run;
      run += v[i];
    }
    __syncthreads();   // part has been read before the next window writes it
    carry = total;
  }
  if (w == 0 && dok) tot[d] = carry;
}

// LDS of the scatter.  Region A: the waves' tag tables during the ranking,
// then the staged block.  Region B: the running counts of wave pairs (wave
// 2p in the low and wave 2p + 1 in the high half of a word) during the
// ranking and the fix-up, then the per-digit global bases G, then the fill.
// Padding: a thread of the fix-up reads 8 consecutive digits (32 bytes) of a
// pair row and a thread of the fill scan 16 consecutive positions (64 bytes);
// 16 bytes of padding after each such group put the lanes of one access on
// different banks.
__device__ __forceinline__ int sort_cidx(int d) { return d + 4 * (d >> 3); }
__device__ __forceinline__ int sort_fidx(int i) { return i + 4 * (i >> 4); }
constexpr int kSortTrash = kSortBinsMax;                             // digit of the empty lanes of a ragged block
constexpr int kSortTagRow = kSortBinsMax + 16;                       // bytes, with the trash digit
constexpr int kSortCntRow = kSortBinsMax + kSortBinsMax / 2 + 4;     // words, padded, with the trash digit
constexpr int kSortFillInts = kSortBlock + kSortBlock / 4;
constexpr int kSortRegionA = (kSortWaves * kSortTagRow > kSortBlock * 4 ? kSortWaves * kSortTagRow : kSortBlock * 4);
constexpr int kSortRegionB = kSortWaves / 2 * kSortCntRow * 4;
static_assert(kSortRegionB >= kSortFillInts * 4 && kSortRegionB >= kSortBinsMax * 4, "G and the fill fit in region B");
static_assert(kSortBlock <= (1 << 13) && kSortDigitBits + 13 <= 31, "staged word: digit << 13 | entry");
static_assert(kSortRounds * 64 < (1 << 16), "a wave's count fits in half a word");

// Stable rank + scatter of one block.  SLOTS: the value is the entry's
// position (pass 0).  FILL (one-pass sort): the sorted experts are written as
// runs from the digit totals, in a coalesced fill of the block's own output
// range, and only the slots are scattered; block 0 writes the offsets.
// Entry e of the block sits at wave w, round r, lane l with
// e = 1024 w + 64 r + l.
template <bool SLOTS, bool FILL>
__global__ __launch_bounds__(kSortThreads) void sort_scatter_kernel(SortPassArgs a) {
  constexpr int R = kSortRounds, W = kSortWaves;
  constexpr int kPer = kSortBinsMax / kSortThreads;   // digits per thread in the fix-up (8)
  constexpr int kFill = kSortBlock / kSortThreads;    // positions per thread in the fill (16)
  __shared__ int4 regA[kSortRegionA / 16];
  __shared__ int4 regB[kSortRegionB / 16];
  __shared__ int wsum[W][2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = sort_chunk(blockIdx.x, a.B);
  const long long base = (long long)c * kSortBlock;
  const int nv = a.n - base < kSortBlock ? (int)(a.n - base) : kSortBlock;
  const bool full = nv == kSortBlock;
  unsigned* cnt = (unsigned*)regB;

  // digit totals and this block's column prefix for digits kPer t .. kPer t + kPer - 1
  const int d0 = threadIdx.x * kPer;
  const int* crow = a.hist + (size_t)c * a.bins;
  int gt[kPer], cp[kPer];
  if ((a.bins & 3) == 0 && d0 + kPer <= a.bins) {
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const int4 x = ((const int4*)(a.tot + d0))[q], y = ((const int4*)(crow + d0))[q];
      gt[4 * q] = x.x, gt[4 * q + 1] = x.y, gt[4 * q + 2] = x.z, gt[4 * q + 3] = x.w;
      cp[4 * q] = y.x, cp[4 * q + 1] = y.y, cp[4 * q + 2] = y.z, cp[4 * q + 3] = y.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int d = d0 + j;
      gt[j] = d < a.bins ? a.tot[d] : 0;
      cp[j] = d < a.bins ? crow[d] : 0;
    }
  }
  for (int i = threadIdx.x; i < kSortRegionB / 16; i += kSortThreads) regB[i] = make_int4(0, 0, 0, 0);
  // digits of the lane's entries (the trash digit past the end of the block)
  const int lbase = w * 64 * R + lane;
  int dg[R];
  if (full) {
#pragma unroll
    for (int r = 0; r < R; ++r) dg[r] = a.keys_in[base + lbase + r * 64];
#pragma unroll
    for (int r = 0; r < R; ++r) dg[r] = sort_digit(dg[r], a);
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = lbase + r * 64;
      dg[r] = e < nv ? sort_digit(a.keys_in[base + e], a) : kSortTrash;
    }
  }
  __syncthreads();

  // ranking.  The wave's LDS operations complete in issue order; the three
  // phases below issue them without waiting in between.
  // (A) every lane writes its lane number into the wave's tag table at its
  //     digit and reads the byte back: lanes of one digit read the same
  //     winner, lanes of different digits different ones.
  uint8_t* tw = (uint8_t*)regA + w * kSortTagRow;
  unsigned* cw = cnt + (w >> 1) * kSortCntRow;
  const int half = 16 * (w & 1);
  int rep[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    tw[dg[r]] = (uint8_t)lane;
    // compiler barrier: the read must go to LDS (other lanes wrote the same
    // byte), not be forwarded from this lane's own store
    asm volatile("" ::: "memory");
    rep[r] = tw[dg[r]];
  }
  // (B) the rank among the lanes sharing a winner (a round where every lane
  //     reads its own number has no repeated digit); the winner adds the
  //     group's size to the wave's running count of the digit and gets the
  //     count before it
  const unsigned long long lt = (1ull << lane) - 1ull;
  int rank[R];
  unsigned old[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const unsigned long long lose = __builtin_amdgcn_ballot_w64(rep[r] != lane);
    int rk = 0, gsize = 1;
    if (lose != 0) {
      if (__builtin_popcountll(lose) <= 8) {
        // few repeated digits: one ballot per group
        unsigned long long todo = lose;
        while (todo != 0) {
          const int r0 = __builtin_amdgcn_readlane(rep[r], __builtin_ctzll(todo));
          const unsigned long long g = __builtin_amdgcn_ballot_w64(rep[r] == r0);
          if (rep[r] == r0) {
            rk = __builtin_popcountll(g & lt);
            gsize = __builtin_popcountll(g);
          }
          todo &= ~g;
        }
      } else {
        // many: match the winners' 6-bit lane numbers
        unsigned long long peers = ~0ull;
#pragma unroll
        for (int bit = 0; bit < 6; ++bit) {
          const bool set = ((rep[r] >> bit) & 1) != 0;
          const unsigned long long bb = __builtin_amdgcn_ballot_w64(set);
          peers &= set ? bb : ~bb;
        }
        rk = __builtin_popcountll(peers & lt);
        gsize = __builtin_popcountll(peers);
      }
    }
    rank[r] = rk;
    old[r] = rep[r] == lane ? atomicAdd(&cw[sort_cidx(dg[r])], (unsigned)gsize << half) : 0u;
  }
  // (C) every lane takes its winner's count
  int pos[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    pos[r] = (int)((__builtin_amdgcn_ds_bpermute(rep[r] << 2, (int)old[r]) >> half) & 0xffff) + rank[r];
  __syncthreads();

  // fix-up per digit: the block's count (sum over the waves), its exclusive
  // prefix over the digits (block-local start) and the global start of
  // (digit, this block) = totals of the digits below + column prefix
  uint4 cr[W / 2][kPer / 4];
#pragma unroll
  for (int u = 0; u < W / 2; ++u)
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) cr[u][q] = ((const uint4*)(cnt + u * kSortCntRow + sort_cidx(d0)))[q];
  auto pw = [&](int u, int j) -> unsigned {   // the pair word of pair row u, digit d0 + j
    const uint4& q = cr[u][j >> 2];
    return (j & 3) == 0 ? q.x : (j & 3) == 1 ? q.y : (j & 3) == 2 ? q.z : q.w;
  };
  int lc[kPer];
  int ls = 0, gs = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    int t = 0;
#pragma unroll
    for (int u = 0; u < W / 2; ++u) t += (int)(pw(u, j) & 0xffff) + (int)(pw(u, j) >> 16);
    lc[j] = t;
    ls += t;
    gs += gt[j];
  }
  const int xl = wave_scan_add(ls), xg = wave_scan_add(gs);
  if (lane == 63) {
    wsum[w][0] = xl;
    wsum[w][1] = xg;
  }
  __syncthreads();
  int bl = xl - ls, bg = xg - gs;
#pragma unroll
  for (int u = 0; u < W; ++u) {
    bl += u < w ? wsum[u][0] : 0;
    bg += u < w ? wsum[u][1] : 0;
  }
  const bool write_offsets = FILL && c == 0;
  int g[kPer], gstart[kPer];
  unsigned st[W / 2][kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (write_offsets && d0 + j < a.bins) a.offsets[d0 + j] = bg;
    gstart[j] = bg;
    g[j] = bg + cp[j] - bl;
    unsigned run = (unsigned)bl;
#pragma unroll
    for (int u = 0; u < W / 2; ++u) {
      const unsigned x = pw(u, j);
      st[u][j] = run | (run + (x & 0xffff)) << 16;   // starts of waves 2u and 2u + 1
      run += (x & 0xffff) + (x >> 16);
    }
    bl += lc[j];
    bg += gt[j];
  }
  if (write_offsets && threadIdx.x == 0) a.offsets[a.bins] = a.n;
#pragma unroll
  for (int u = 0; u < W / 2; ++u)
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q)
      ((uint4*)(cnt + u * kSortCntRow + sort_cidx(d0)))[q] =
          make_uint4(st[u][4 * q], st[u][4 * q + 1], st[u][4 * q + 2], st[u][4 * q + 3]);
  __syncthreads();

  // stage the block in LDS in (digit, entry) order
  int* stg = (int*)regA;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = lbase + r * 64;
    if (full || e < nv) {
      const int start = (int)((cw[sort_cidx(dg[r])] >> half) & 0xffff);
      stg[(start + pos[r]) & (kSortBlock - 1)] = dg[r] << 13 | e;   // < nv by construction
    }
  }
  __syncthreads();
  int* G = (int*)regB;
#pragma unroll
  for (int q = 0; q < kPer / 4; ++q) ((int4*)(G + d0))[q] = make_int4(g[4 * q], g[4 * q + 1], g[4 * q + 2], g[4 * q + 3]);
  __syncthreads();
  // write it out: consecutive lanes on consecutive positions of each digit's run
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = threadIdx.x + kSortThreads * r;
    if (i < nv) {
      const int x = stg[i];
      const int e = x & (kSortBlock - 1);
      // p < n by construction; the clamp keeps every store inside the outputs
      const int p = min((unsigned)(G[x >> 13] + i), (unsigned)(a.n - 1));
      if (!FILL) a.keys_out[p] = a.keys_in[base + e];
      a.vals_out[p] = SLOTS ? (int)(base + e) : a.vals_in[base + e];
    }
  }
  if (!FILL) return;

  // the sorted experts of output positions base .. base + nv - 1: a mark at
  // the start of every digit run beginning there (and at 0 the digit whose
  // run covers base), then a running maximum
  __syncthreads();
  int* F = (int*)regB;
  for (int i = threadIdx.x; i < kSortFillInts / 4; i += kSortThreads) ((int4*)F)[i] = make_int4(-1, -1, -1, -1);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int d = d0 + j;
    if (d < a.bins && gt[j] > 0) {
      const long long s0 = gstart[j];
      if (s0 >= base && s0 < base + nv) F[sort_fidx((int)(s0 - base))] = d;
      else if (s0 < base && s0 + gt[j] > base) F[0] = d;
    }
  }
  __syncthreads();
  int fv[kFill];
  int* Ft = F + sort_fidx(kFill * threadIdx.x);
#pragma unroll
  for (int q = 0; q < kFill / 4; ++q) {
    const int4 x = ((const int4*)Ft)[q];
    fv[4 * q] = x.x, fv[4 * q + 1] = x.y, fv[4 * q + 2] = x.z, fv[4 * q + 3] = x.w;
  }
#pragma unroll
  for (int j = 1; j < kFill; ++j) fv[j] = max(fv[j], fv[j - 1]);
  const int xm = wave_scan_max(fv[kFill - 1]);
  if (lane == 63) wsum[w][0] = xm;
  __syncthreads();
  int before = __shfl_up(xm, 1);
  if (lane == 0) before = -1;
#pragma unroll
  for (int u = 0; u < W; ++u) before = u < w ? max(before, wsum[u][0]) : before;
#pragma unroll
  for (int q = 0; q < kFill / 4; ++q)
    ((int4*)Ft)[q] = make_int4(max(fv[4 * q], before), max(fv[4 * q + 1], before), max(fv[4 * q + 2], before),
                               max(fv[4 * q + 3], before));
  __syncthreads();
  int* out = a.keys_out + base;
  if (full) {
#pragma unroll
    for (int q = 0; q < kFill / 4; ++q) {
      const int i4 = q * kSortThreads + threadIdx.x;
      ((int4*)out)[i4] = *(const int4*)(F + sort_fidx(4 * i4));
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = threadIdx.x + kSortThreads * r;
      if (i < nv) out[i] = F[sort_fidx(i)];
    }
  }
}

// offsets[e] = first position whose expert is >= e: thread i (0..n) looks at
// the pair (keys[i-1], keys[i]) (keys[-1] = -1, keys[n] = M) and writes every e
// in (keys[i-1], keys[i]]; the ranges are disjoint and cover 0..M.
__global__ __launch_bounds__(256) void sort_offsets_kernel(SortOffsetsArgs a) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i > a.n) return;
  int prev = i > 0 ? a.keys[i - 1] : -1;
  int cur = i < a.n ? a.keys[i] : a.M;
  prev = prev < -1 ? -1 : prev;          // out-of-range experts write nothing outside 0..M
  cur = cur > a.M ? a.M : cur;
  for (int e = prev + 1; e <= cur; ++e) a.offsets[e] = (int)i;
}

hipError_t launch_dispatch_sort(const int* idx, int n, int M, int* sorted_expert, int* sorted_slot,
                                int* offsets, int* hist, int* tmp_keys, int* tmp_vals, hipStream_t stream) {
  const int P = sort_passes(M);
  const int B = (int)sort_blocks(n);
  const int* kin = idx;
  const int* vin = nullptr;
  for (int p = 0; p < P; ++p) {
    const bool to_out = ((P - 1 - p) & 1) == 0;
    SortPassArgs a;
    a.keys_in = kin;
    a.vals_in = vin;
    a.keys_out = to_out ? sorted_expert : tmp_keys;
    a.vals_out = to_out ? sorted_slot : tmp_vals;
    a.bins = sort_bins(M, p, P);
    a.hist = hist;
    a.tot = hist + (size_t)B * a.bins;
    a.offsets = P == 1 ? offsets : nullptr;
    a.n = n;
    a.B = B;
    a.shift = p * kSortDigitBits;
    a.mask = p < P - 1 ? (unsigned)(kSortBinsMax - 1) : 0xffffffffu;
    hipLaunchKernelGGL(sort_count_kernel, dim3((unsigned)B), dim3(kSortCountThreads), 0, stream, a);
    hipLaunchKernelGGL(sort_colscan_kernel, dim3((unsigned)((a.bins + 63) / 64)), dim3(kSortColWaves * 64), 0, stream,
                       a.hist, a.tot, B, a.bins);
    if (P == 1)
      hipLaunchKernelGGL((sort_scatter_kernel<true, true>), dim3((unsigned)B), dim3(kSortThreads), 0, stream, a);
    else if (p == 0)
      hipLaunchKernelGGL((sort_scatter_kernel<true, false>), dim3((unsigned)B), dim3(kSortThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((sort_scatter_kernel<false, false>), dim3((unsigned)B), dim3(kSortThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    kin = a.keys_out;
    vin = a.vals_out;
  }
  if (P == 1) return hipSuccess;
  SortOffsetsArgs o;
  o.keys = sorted_expert;
  o.offsets = offsets;
  o.n = n;
  o.M = M;
  hipLaunchKernelGGL(sort_offsets_kernel, dim3((unsigned)(((long long)n + 1 + 255) / 256)), dim3(256), 0, stream, o);
  return hipGetLastError();
}

}  // namespace more
