// Template instances: full-rank router, both storage types and gates.
#include "more_dispatch.h"
namespace more {
template <int DT, bool FULL>
static fullrank_fn pick_fr(int kmax) {
  switch (kmax) {
    case 4: return fullrank_kernel<DT, 4, FULL, waves_for_kmax(4)>;
    case 8: return fullrank_kernel<DT, 8, FULL, waves_for_kmax(8)>;
    case 16: return fullrank_kernel<DT, 16, FULL, waves_for_kmax(16)>;
    default: return fullrank_kernel<DT, 32, FULL, waves_for_kmax(32)>;
  }
}
fullrank_fn pick_fullrank(int dt, bool full, int kmax) {
  if (dt == 0) return full ? pick_fr<0, true>(kmax) : pick_fr<0, false>(kmax);
  return full ? pick_fr<1, true>(kmax) : pick_fr<1, false>(kmax);
}
}  // namespace more
