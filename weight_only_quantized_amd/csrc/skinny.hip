// Host launcher of the skinny family (kernels and per-width dispatch: skinny_impl.h).
#include <hip/hip_runtime.h>

#include "skinny_impl.h"

namespace gq {

bool skinny_needs_xsorted(const gptq_layer* L, int64_t M) {
  return L->has_perm && (!x_fits_lds(M, L->Kp) || !L->iperm);
}

hipError_t launch_skinny(const GemmCall& c) {
  const gptq_layer* L = c.L;
  if (uses_mid(L, c.M)) return launch_mid(c);
  SkinnyArgs a;
  a.wq = L->wq;
  a.meta = L->meta;
  a.scale32 = L->scale32;
  a.y = reinterpret_cast<uint16_t*>(c.y);
  a.M = (int)c.M; a.K = L->K; a.Kp = L->Kp; a.N = L->N; a.KC = L->KC; a.CT = L->CT; a.G = L->G;
  a.Kx = L->Kp;
  a.cgs = 1;
  segment_divisor(L, &a.gmagic, &a.gshift);
  a.scale_kind = L->scales_dtype;
  a.bias = c.bias;
  a.iperm = nullptr;
  if (skinny_needs_xsorted(L, c.M)) {
    hipError_t e = launch_prep(c, false);
    if (e != hipSuccess) return e;
    a.x = reinterpret_cast<const uint16_t*>(c.ws);
    a.ld = L->Kp;
  } else {
    a.x = reinterpret_cast<const uint16_t*>(c.x);
    a.ld = L->K;
    if (L->has_perm) a.iperm = L->iperm;   // scattered into sorted order while staging x in LDS
  }
  switch (L->bits) {
    case 2: return skinny_b2(a, c.x_bf16, L->seg_steps, c.stream);
    case 3: return skinny_b3(a, c.x_bf16, L->seg_steps, c.stream);
    case 4: return skinny_b4(a, c.x_bf16, L->seg_steps, c.stream);
    case 5: return skinny_b5(a, c.x_bf16, L->seg_steps, c.stream);
    case 6: return skinny_b6(a, c.x_bf16, L->seg_steps, c.stream);
    case 7: return skinny_b7(a, c.x_bf16, L->seg_steps, c.stream);
    default: return skinny_b8(a, c.x_bf16, L->seg_steps, c.stream);
  }
}

}  // namespace gq
