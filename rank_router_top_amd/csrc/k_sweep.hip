// Template instances: the expert sweep with the up-projection tiles shared
// through LDS (more_sweep.h), for k <= 4 or <= 8 and r <= 16, 32, 64.
#include "more_dispatch.h"
namespace more {
// ring slots per rank block count (LDS: RING tiles of R16 KiB + 256 B, then
// the consumers' logs and result blocks)
template <int R16> struct SwRing { static constexpr int value = R16 >= 4 ? 8 : 16; };
template <int KMAX> struct SwCap { static constexpr int value = KMAX <= 4 ? 8 : 10; };

template <int KMAX, int R16, bool LSE, bool FULL>
static sweep_fn sw_inst() {
  return sweep_kernel<KMAX, R16, LSE, FULL, kSwCons, SwRing<R16>::value, SwCap<KMAX>::value>;
}
template <int KMAX, bool LSE, bool FULL>
static sweep_fn sw_r(int r16) {
  switch (r16) {
    case 1: return sw_inst<KMAX, 1, LSE, FULL>();
    case 2: return sw_inst<KMAX, 2, LSE, FULL>();
    default: return sw_inst<KMAX, 4, LSE, FULL>();
  }
}
sweep_fn pick_sweep(bool full, bool lse, int kmax, int r16) {
  if (full) return kmax <= 4 ? sw_r<4, true, true>(r16) : sw_r<8, true, true>(r16);
  if (lse) return kmax <= 4 ? sw_r<4, true, false>(r16) : sw_r<8, true, false>(r16);
  return kmax <= 4 ? sw_r<4, false, false>(r16) : sw_r<8, false, false>(r16);
}
template <int KMAX>
static size_t sw_bytes(int r16) {
  switch (r16) {
    case 1: return SwLds<1, kSwCons, SwRing<1>::value, SwCap<KMAX>::value, KMAX>::bytes;
    case 2: return SwLds<2, kSwCons, SwRing<2>::value, SwCap<KMAX>::value, KMAX>::bytes;
    default: return SwLds<4, kSwCons, SwRing<4>::value, SwCap<KMAX>::value, KMAX>::bytes;
  }
}
size_t sweep_lds_bytes(int kmax, int r16) { return kmax <= 4 ? sw_bytes<4>(r16) : sw_bytes<8>(r16); }
}  // namespace more
