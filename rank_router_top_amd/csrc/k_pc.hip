// Template instances: producer/consumer low-rank router (bf16, k <= 8, r <= 64).
#include "more_dispatch.h"
namespace more {
template <int KMAX>
static size_t lds_r(int r16, long long mpad) {
  switch (r16) {
    case 1: return PcLds<KMAX, 1>::bytes(mpad);
    case 2: return PcLds<KMAX, 2>::bytes(mpad);
    case 4: return PcLds<KMAX, 4>::bytes(mpad);
    default: return 0;
  }
}
size_t pc_lds_bytes(int kmax, int r16, long long mpad) {
  if (!pc_shape_ok(kmax, r16, mpad)) return 0;
  return kmax <= 4 ? lds_r<4>(r16, mpad) : lds_r<8>(r16, mpad);
}
template <bool FULL, int KMAX, bool TAIL>
static pc_fn pick_r(int r16) {
  switch (r16) {
    case 1: return pc_kernel<KMAX, FULL, 1, pc_depth(1, TAIL), TAIL>;
    case 2: return pc_kernel<KMAX, FULL, 2, pc_depth(2, TAIL), TAIL>;
    default: return pc_kernel<KMAX, FULL, 4, pc_depth(4, TAIL), TAIL>;
  }
}
template <bool FULL, bool TAIL>
static pc_fn pick_k(int kmax, int r16) {
  return kmax <= 4 ? pick_r<FULL, 4, TAIL>(r16) : pick_r<FULL, 8, TAIL>(r16);
}
pc_fn pick_pc(bool full, int kmax, int r16, bool tail) {
  if (full) return tail ? pick_k<true, true>(kmax, r16) : pick_k<true, false>(kmax, r16);
  return tail ? pick_k<false, true>(kmax, r16) : pick_k<false, false>(kmax, r16);
}
}  // namespace more
