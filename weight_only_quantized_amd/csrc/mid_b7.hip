// Instantiation unit of the mid family for 7-bit codes (kernel in mid_impl.h).
#include "mid_impl.h"

namespace gq {
hipError_t mid_b7(const MidArgs& a, const MidPlan& p, int x_bf16, int seg, hipStream_t s) {
  return mid_bits<7>(a, p, x_bf16, seg, s);
}
}  // namespace gq
