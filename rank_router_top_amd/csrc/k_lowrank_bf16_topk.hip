// Template instances: low-rank router, bf16 storage, top-k-softmax gate.
#include "more_dispatch.h"
namespace more {
lowrank_fn pick_lowrank_bf16_topk(int kmax, int r16) { return pick_lowrank_k<0, false>(kmax, r16); }
}  // namespace more
