// more_sort.h -- expert dispatch after the router: sort + count.
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. E, Fig. 9: the router's (N, k) expert indices become the N k
// slots ordered by expert plus the offset of each expert's run, which is what
// a grouped expert GEMM consumes.  Slot s = n k + j; slots of one expert stay
// in increasing s (stable), offsets[e] = first position of expert e,
// offsets[M] = N k.
//
// Design (HBM-bound, no MFMA work): a counting sort on 12-bit digits of the
// expert index -- one pass for M <= 4096 (the digit is the expert itself),
// LSD passes of 12 bits beyond.  The entries are cut into blocks of 8192;
// each pass is three kernels:
//   sort_count_kernel    per-block digit counts (LDS atomics; order does not
//                        matter for a count), written block-major:
//                        hist[b * bins + d];
//   sort_colscan_kernel  per digit, the exclusive prefix of its counts over
//                        the blocks (in place) and its total;
//   sort_scatter_kernel  each block ranks its entries stably within each
//                        digit, stages them in LDS in (digit, entry) order and
//                        writes them to (digits below, summed over all
//                        blocks) + (this digit in earlier blocks) + rank.
// The stable rank inside a wave round of 64 entries: every lane writes its
// lane number into a per-wave table at its digit and reads it back; lanes
// with equal digits read the same winner, lanes with different digits
// different ones.  A round where every lane reads its own number has no
// repeated digit (the common case for many experts); otherwise the lanes
// sharing a winner are grouped by ballots over the winner's 6-bit lane
// number (or, for a few groups, one ballot per group).  The winner adds the
// group's size to the wave's running count of the digit with an LDS atomic
// that returns the count before it, and the group reads it from the winner
// lane.  Waves own consecutive ranges of the block, so (wave, round, lane) is
// entry order.
// For M <= 4096 the slots are the only scattered output: each block writes
// the sorted experts of its own output range as runs read off the digit
// totals (a coalesced fill), and block 0 writes the offsets.  After several
// passes sort_offsets_kernel reads the sorted experts once.
// Blocks are spread so that each XCD (blocks are dealt round-robin to the 8
// XCDs) owns a contiguous range of entries: an expert's run is then written
// in 8 contiguous pieces, one per XCD's L2.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace more {

constexpr int kSortThreads = 512;                        // scatter: 8 waves
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortRounds = 16;                          // entries per lane
constexpr int kSortBlock = kSortThreads * kSortRounds;   // 8192 entries per block
constexpr int kSortCountThreads = 1024;                  // count: 8 entries per thread
constexpr int kSortDigitBits = 12;
constexpr int kSortBinsMax = 1 << kSortDigitBits;        // 4096
constexpr int kSortColWaves = 16;                        // column scan: 1024 threads

// Passes for expert indices in [0, M): 12 bits each (at least one).
inline int sort_passes(long long M) {
  int bits = 0;
  while (bits < 31 && (1LL << bits) < M) ++bits;
  return bits <= kSortDigitBits ? 1 : (bits + kSortDigitBits - 1) / kSortDigitBits;
}

// Digit bins of pass p of P: 4096 before the last pass; the last pass covers
// the remaining high bits of M - 1 (for one pass: M itself).
inline int sort_bins(long long M, int p, int P) {
  if (p < P - 1) return kSortBinsMax;
  return (int)(((M - 1) >> (kSortDigitBits * p)) + 1);
}

// Blocks of n entries.
inline long long sort_blocks(long long n) { return (n + kSortBlock - 1) / kSortBlock; }

// ints of the count matrix + digit totals for n entries (the largest pass).
inline size_t sort_hist_ints(long long n, long long M) {
  const long long B = sort_blocks(n) > 0 ? sort_blocks(n) : 1;
  const long long bins = M < kSortBinsMax ? M : kSortBinsMax;
  return (size_t)((B + 1) * bins);
}

struct SortPassArgs {
  const int* keys_in;   // n expert indices (pass 0: the router's output)
  const int* vals_in;   // n slot numbers; null in pass 0 (the slot is the position)
  int* keys_out;
  int* vals_out;
  int* hist;            // [B][bins] counts -> exclusive prefix over the blocks
  int* tot;             // [bins] digit totals
  int* offsets;         // one-pass sort: the M + 1 offsets (block 0 writes them); else null
  int n, B;
  int shift;            // digit = ((key >> shift) & mask), clamped to bins - 1
  unsigned mask;
  int bins;
};

struct SortOffsetsArgs {
  const int* keys;      // n sorted expert indices
  int* offsets;         // M + 1
  int n, M;
};

// Enqueues every kernel of the sort on `stream`: passes P over (idx ->
// ... -> sorted_expert, sorted_slot) with tmp_keys / tmp_vals between passes
// (null for one pass), then the offsets.  hist holds sort_hist_ints(n, M) ints.
hipError_t launch_dispatch_sort(const int* idx, int n, int M, int* sorted_expert, int* sorted_slot,
                                int* offsets, int* hist, int* tmp_keys, int* tmp_vals, hipStream_t stream);

}  // namespace more
