// more_merge.h -- merge of per-shard top-k candidate lists (experts sharded).
//
// Method: "MoRE: Scaling mixture of experts with hardware-aware low-rank
// routing", App. E.3 (top-k over expert shards as a hierarchical merge) with
// the gates of Fig. 12 and eq. (6) / (8).  With the M experts cut into G
// shards of W consecutive experts (the last may be shorter), shard g routes
// every token over its own experts and hands over its k best (logit, local
// index) pairs, ordered by (logit desc, index asc), and for eq. (6) its
// log-sum-exp over its experts.  The token's top k over all M experts are
// the k best of the G k candidates (a global top-k entry is in its shard's
// top k); the full-softmax normaliser is the log-sum-exp of the G shard
// values.  One lane per token merges the G sorted lists.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace more {

struct MergeArgs {
  const float* cand_logit;   // [G][N][k]
  const int* cand_idx;       // [G][N][k] shard-local
  const float* shard_lse;    // [G][N] (full-softmax gates) or null
  int* out_idx;
  float* out_gate;
  float* out_logit;
  float* out_lse;
  long long N, W;
  int G, k;
};

hipError_t launch_topk_merge(const MergeArgs& a, bool full, hipStream_t stream);

}  // namespace more
