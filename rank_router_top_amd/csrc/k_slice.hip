// Template instances: expert-slice low-rank router (bf16, r in {16, 32}, M = 4096, k <= 8).
// The packed bias is zero when the caller gave none, so every instance reads it.
#include "more_dispatch.h"
namespace more {
// R2 tiles per consumer kept in VGPRs (the rest of the 16 live in LDS) and
// z-ring slots, chosen so that the VGPRs stay within 168 (three waves per
// SIMD) and the LDS within 160 KiB: all 16 tiles at r = 16; 9 tiles with a
// 2-slot ring at r = 32 (10 tiles and 3 slots in the full-softmax mode, whose
// per-token normalisers take 8 KiB of LDS).
constexpr int sl_tv(bool full, int r16) { return r16 == 1 ? 16 : full ? 10 : 9; }
constexpr int sl_nz(bool full, int r16) { return r16 == 1 ? 3 : full ? 3 : 2; }
template <bool FULL, int R16>
static size_t lds_of() { return SlLds<FULL, true, R16, sl_tv(FULL, R16), sl_nz(FULL, R16)>::bytes; }
size_t slice_lds_bytes(bool full, int r16) {
  if (r16 == 1) return full ? lds_of<true, 1>() : lds_of<false, 1>();
  if (r16 == 2) return full ? lds_of<true, 2>() : lds_of<false, 2>();
  return 0;
}
template <bool FULL, int R16>
static slice_fn pick_t(bool tail) {
  constexpr int TV = sl_tv(FULL, R16), NZ = sl_nz(FULL, R16);
  if (tail) return slice_kernel<FULL, true, R16, TV, NZ, pc_depth(R16, true), true>;
  return slice_kernel<FULL, true, R16, TV, NZ, pc_depth(R16, false), false>;
}
slice_fn pick_slice(bool full, int r16, bool tail) {
  if (r16 == 1) return full ? pick_t<true, 1>(tail) : pick_t<false, 1>(tail);
  if (r16 == 2) return full ? pick_t<true, 2>(tail) : pick_t<false, 2>(tail);
  return nullptr;
}
}  // namespace more
