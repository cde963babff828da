// more_sort.h -- expert dispatch after the router: sort + count.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. E, Fig. 9: the router's (N, k) expert indices become the N k
// slots ordered by expert plus the offset of each expert's run, which is what
// a grouped expert GEMM consumes.  Slot s = n k + j; slots of one expert stay
// in increasing s (stable), offsets[e] = first position of expert e,
// offsets[M] = N k.
//
// Design (HBM-bound, no MFMA work): an LSD radix sort on 6-bit digits of the
// expert index (two passes for M <= 4096), each pass three kernels:
//   sort_hist_kernel     per-block digit histogram (64 bins; one LDS atomic
//                        per group of equal digits in a wave round),
//                        written digit-major: hist[d * B + b];
//   sort_scan_kernel     one workgroup per digit: exclusive scan of row d of
//                        hist and its total; the scatter adds the totals of
//                        the digits below -> the first output position of
//                        digit d's elements from block b;
//   sort_scatter_kernel  the block's elements are ranked stably within the
//                        block with wave ballots (a 64-way multisplit: six
//                        ballots give each lane the mask of lanes with its
//                        digit) and a per-wave running count per digit in LDS,
//                        then written to base + rank.
// Element e of block b sits at wave w, round r, lane l with
// e = b C + w 64 R + r 64 + l, so loads are coalesced and the ranking order
// (wave, round, lane) is the element order: every pass is stable.
// sort_offsets_kernel then reads the sorted experts once and writes each
// expert's start where the run changes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace more {

constexpr int kSortThreads = 256;                 // 4 waves
constexpr int kSortRounds = 16;                   // elements per lane
constexpr int kSortBlock = kSortThreads * kSortRounds;   // elements per block
constexpr int kSortDigitBits = 6;
constexpr int kSortBuckets = 1 << kSortDigitBits;
constexpr int kSortScanThreads = 1024;

// Passes for expert indices in [0, M): 6 bits each (at least one).
inline int sort_passes(long long M) {
  int bits = 0;
  while (bits < 31 && (1LL << bits) < M) ++bits;
  return bits <= kSortDigitBits ? 1 : (bits + kSortDigitBits - 1) / kSortDigitBits;
}

struct SortPassArgs {
  const int* keys_in;   // n expert indices (pass 0: the router's output)
  const int* vals_in;   // n slot numbers; null in pass 0 (the slot is the position)
  int* keys_out;
  int* vals_out;
  int* hist;            // [64][B]
  const int* tot;       // [64] row totals of hist
  int n, B, shift;
};

struct SortOffsetsArgs {
  const int* keys;      // n sorted expert indices
  int* offsets;         // M + 1
  int n, M;
};

// Enqueues every kernel of the sort on `stream`: passes P over (idx ->
// ... -> sorted_expert, sorted_slot) with tmp_keys / tmp_vals between passes,
// then the offsets.  hist holds 64 B + 64 ints (counts, then row totals).
hipError_t launch_dispatch_sort(const int* idx, int n, int M, int* sorted_expert, int* sorted_slot,
                                int* offsets, int* hist, int* tmp_keys, int* tmp_vals, hipStream_t stream);

}  // namespace more
