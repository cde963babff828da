// Template instances: low-rank router, fp32 storage, both gates.
#include "more_dispatch.h"
namespace more {
lowrank_fn pick_lowrank_f32(bool full, int kmax, int r16) {
  return full ? pick_lowrank_k<1, true>(kmax, r16) : pick_lowrank_k<1, false>(kmax, r16);
}
}  // namespace more
