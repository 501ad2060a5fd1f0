// Instantiation unit of the mid family for 8-bit codes (kernel in mid_impl.h).
#include "mid_impl.h"

namespace gq {
hipError_t mid_b8(const MidArgs& a, const MidPlan& p, int x_bf16, int seg, hipStream_t s) {
  return mid_bits<8>(a, p, x_bf16, seg, s);
}
}  // namespace gq
