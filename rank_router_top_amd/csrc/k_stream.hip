// Template instances: persistent streaming low-rank router (bf16, r <= 64).
#include "more_dispatch.h"
namespace more {
template <bool FULL, int KMAX>
static stream_fn pick_r(int r16) {
  constexpr int W = waves_for_kmax(KMAX);
  switch (r16) {
    case 1: return stream_kernel<KMAX, FULL, 1, stream_depth(1), W>;
    case 2: return stream_kernel<KMAX, FULL, 2, stream_depth(2), W>;
    default: return stream_kernel<KMAX, FULL, 4, stream_depth(4), W>;
  }
}
template <bool FULL>
static stream_fn pick_k(int kmax, int r16) {
  switch (kmax) {
    case 4: return pick_r<FULL, 4>(r16);
    case 8: return pick_r<FULL, 8>(r16);
    case 16: return pick_r<FULL, 16>(r16);
    default: return pick_r<FULL, 32>(r16);
  }
}
stream_fn pick_stream(bool full, int kmax, int r16) {
  return full ? pick_k<true>(kmax, r16) : pick_k<false>(kmax, r16);
}
}  // namespace more
