// Template instances: split-M router (few tokens, many experts), projection
// and the top-k-softmax routing instances.
#include "more_dispatch.h"
namespace more {
splitm_proj_fn pick_splitm_proj(int r16) {
  switch (r16) {
    case 1: return splitm_proj_kernel<1>;
    case 2: return splitm_proj_kernel<2>;
    case 4: return splitm_proj_kernel<4>;
    default: return splitm_proj_kernel<8>;
  }
}
splitm_fn pick_splitm_topk(int kmax, int r16) { return pick_splitm_k<false>(kmax, r16); }
}  // namespace more
