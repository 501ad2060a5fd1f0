// Instantiation unit of the skinny family for 6-bit codes (kernels are in skinny_impl.h).
#include "skinny_impl.h"

namespace gq {
hipError_t skinny_b6(const SkinnyArgs& a, int x_bf16, int seg, hipStream_t s) { return skinny_bits<6>(a, x_bf16, seg, s); }
}  // namespace gq
