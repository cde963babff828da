// Template instances: workgroup-lockstep low-rank router (bf16, k <= 8, r <= 64).
#include "more_dispatch.h"
namespace more {
template <bool FULL, int KMAX, int R16>
static lock_fn inst(size_t* lds) {
  *lds = LockLds<KMAX, R16, kLockKPBM, kLockTPBM>::total;
  return lock_kernel<KMAX, FULL, R16, kLockKPBM, kLockTPBM>;
}
template <bool FULL, int KMAX>
static lock_fn pick_r(int r16, size_t* lds) {
  switch (r16) {
    case 1: return inst<FULL, KMAX, 1>(lds);
    case 2: return inst<FULL, KMAX, 2>(lds);
    default: return inst<FULL, KMAX, 4>(lds);
  }
}
lock_fn pick_lock(bool full, int kmax, int r16, size_t* lds) {
  if (full) return kmax <= 4 ? pick_r<true, 4>(r16, lds) : pick_r<true, 8>(r16, lds);
  return kmax <= 4 ? pick_r<false, 4>(r16, lds) : pick_r<false, 8>(r16, lds);
}
}  // namespace more
