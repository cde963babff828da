// Template instances: two-kernel low-rank router (projection + routing).
#include "more_dispatch.h"
namespace more {
template <bool TAIL>
static proj_fn proj_r(int r16) {
  switch (r16) {
    case 1: return proj_kernel<1, proj_depth(1), TAIL, kProjWaves>;
    case 2: return proj_kernel<2, proj_depth(2), TAIL, kProjWaves>;
    default: return proj_kernel<4, proj_depth(4), TAIL, kProjWaves>;
  }
}
proj_fn pick_proj(int r16, bool tail) { return tail ? proj_r<true>(r16) : proj_r<false>(r16); }
size_t proj_lds_bytes(int r16, int ksp) {
  switch (r16) {
    case 1: return PjLds<1, kProjWaves>::bytes(ksp);
    case 2: return PjLds<2, kProjWaves>::bytes(ksp);
    default: return PjLds<4, kProjWaves>::bytes(ksp);
  }
}
template <bool FULL, bool LSE, int KMAX>
static route_fn route_r(int r16) {
  switch (r16) {
    case 1: return route_kernel<KMAX, FULL, 1, kRouteWaves, LSE>;
    case 2: return route_kernel<KMAX, FULL, 2, kRouteWaves, LSE>;
    default: return route_kernel<KMAX, FULL, 4, kRouteWaves, LSE>;
  }
}
route_fn pick_route(bool full, bool lse, int kmax, int r16) {
  if (full) return kmax <= 4 ? route_r<true, true, 4>(r16) : route_r<true, true, 8>(r16);
  if (lse) return kmax <= 4 ? route_r<false, true, 4>(r16) : route_r<false, true, 8>(r16);
  return kmax <= 4 ? route_r<false, false, 4>(r16) : route_r<false, false, 8>(r16);
}
size_t route_lds_bytes(int kmax, long long mpad) {
  return kmax <= 4 ? RouteLds<4>::bytes(kRouteWaves, mpad) : RouteLds<8>::bytes(kRouteWaves, mpad);
}
}  // namespace more
