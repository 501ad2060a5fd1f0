// Library-internal declarations shared by the host API and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gptq_mi355x.h"
#include "layout.h"

#define GQ_MAGIC 0x47505451u  // "GPTQ"

struct gptq_layer {
  uint32_t magic;
  int device;
  int K, N, bits, group_size, gs_eff, G, Kp, KC, CT;
  int scales_dtype;   // gptq_dtype of the stored scales
  int has_perm;       // 1 when the sorted order is not the identity
  int seg_steps;      // MFMA K steps (of 32) per scale-fixup segment: 4 or 1
  uint32_t* wq;       // runtime words, CT * KC * 64 * bits
  void* scales_rt;    // [CT][G][16] of uint16 (f16/bf16 bits) or uint32 (f32)
  uint8_t* zeros_rt;  // [CT][G][16] stored zeros
  int32_t* perm;      // [Kp]: original input index at each sorted position (-1 = padding)
  int64_t bytes;
};

namespace gq {

// Set the calling thread's last HIP error and return GPTQ_E_HIP.
gptq_status hip_fail(hipError_t e);

// Repack kernels (repack.hip).
hipError_t launch_repack(const gptq_layer* L, const int32_t* qweight, const int32_t* qzeros,
                         const void* scales, hipStream_t s);

// Parameters of one gptq_gemm call as the launchers see them.
struct GemmCall {
  const gptq_layer* L;
  const void* x;      // [M, K] original order
  int64_t M;
  int x_bf16;         // 0 = f16, 1 = bf16
  void* y;
  void* ws;           // workspace base (256-B aligned) or NULL
  size_t ws_bytes;
  hipStream_t stream;
};

// Workspace layout helpers (tiled.hip): sizes in bytes, 256-B aligned parts.
size_t ws_xsorted_bytes(const gptq_layer* L, int64_t M);
size_t ws_nsb_bytes(const gptq_layer* L, int64_t M);
bool needs_nsb(const gptq_layer* L, int x_bf16);   // the tiled family's bias-correction table

// Family launchers.  Both assume the call was validated.
hipError_t launch_skinny(const GemmCall& c);
hipError_t launch_tiled(const GemmCall& c);
// x -> sorted copy (act-order) and/or per-segment sums of x times -bias (tiled family).
hipError_t launch_prep(const GemmCall& c, bool write_xsorted, bool write_nsb);

constexpr int64_t kSkinnyMaxM = 64;

}  // namespace gq
