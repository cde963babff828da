// Template instances: split-M router (few tokens, many experts), full-softmax gate.
#include "more_dispatch.h"
namespace more {
splitm_fn pick_splitm_full(int kmax, int r16) { return pick_splitm_k<true>(kmax, r16); }
}  // namespace more
