// Template instances: low-rank router, bf16 storage, full-softmax gate.
#include "more_dispatch.h"
namespace more {
lowrank_fn pick_lowrank_bf16_full(int kmax, int r16) { return pick_lowrank_k<0, true>(kmax, r16); }
}  // namespace more
