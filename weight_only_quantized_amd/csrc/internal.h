// Library-internal declarations shared by the host API and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gptq_mi355x.h"
#include "layout.h"

struct gptq_layer {
  int device;
  int K, N, bits, group_size, gs_eff, G, Kp, KC, CT;   // bits: runtime code width (2..8)
  int ckpt_bits;      // the checkpoint's code width (equal to bits: every width has its runtime layout)
  int scales_dtype;   // gptq_dtype of the stored scales
  int has_perm;       // 1 when the sorted order is not the identity
  int seg_steps;      // MFMA K steps (of 32) per scale-fixup segment: 4 or 1
  uint32_t* wq;       // runtime words, CT * KC * 64 * bits
  uint32_t* meta;     // [CT][G][16]: 16-bit scale bits | stored zero << 16 (see layout.h)
  uint32_t* scale32;  // [CT][G][16] f32 scale bits when scales_dtype is F32, else NULL
  int32_t* perm;      // [Kp]: original input index at each sorted position (-1 = padding)
  uint16_t* iperm;    // [K]: sorted position of each original input (act-order with Kp <= 8192
                      // only): the skinny kernel scatters x through it into LDS, the prep into
                      // the workspace copy
  int64_t bytes;
};

namespace gq {

// Set the calling thread's last HIP error and return GPTQ_E_HIP.
gptq_status hip_fail(hipError_t e);

// Repack kernels (repack.hip), by how the checkpoint encodes codes and zeros:
enum RepackSource {
  kSrcGptq = 0,        // continuous words, v1 zeros (stored = zero - 1)
  kSrcAwqGemm = 1,     // AutoAWQ GEMM: 4-bit fields along the output dimension, zeros as stored
  kSrcGptqV2 = 2,      // continuous words, zeros as stored
  kSrcGptqPlanar = 3,  // GPTQ_P planar words, v1 zeros
};
hipError_t launch_repack(const gptq_layer* L, const int32_t* qweight, const int32_t* qzeros,
                         const void* scales, RepackSource src, hipStream_t s);

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
  const void* bias;   // [N] in the scales' dtype, or NULL
};

// Workspace layout helpers (tiled.hip): sizes in bytes, 256-B aligned parts.
size_t ws_xsorted_bytes(const gptq_layer* L, int64_t M);
size_t ws_rowexp_bytes(int64_t M);
// the tiled family reads a prepared copy of x: act-order layers, bf16 activations (fp16 copy), and
// K not a multiple of 128 (zero-padded rows)
bool tiled_needs_xsorted(const gptq_layer* L, int x_bf16);

// True when the skinny family needs a sorted copy of x in the workspace (act-order with x too
// large to gather into LDS).
bool skinny_needs_xsorted(const gptq_layer* L, int64_t M);

// The SKINNY path (M <= 64) runs the skinny kernel when one of its forms takes the call and the
// mid kernel (split K, mid.hip) otherwise; the mid kernel's partial sums need workspace.
bool uses_mid(const gptq_layer* L, int64_t M);
// The skinny kernel takes these M > 1 rows in one launch: x read from L2 per chunk, or the
// workgroup's copy of x in LDS (mid.hip; the rules are skinny_impl.h's).
bool skinny_one_launch(const gptq_layer* L, int64_t M);
// K slices the mid kernel would cut a call into (mid.hip), and chunks per K slice of the tiled
// plan (tiled.hip): the inputs of PATH_AUTO between 17 and 32 rows.
int mid_slices(const gptq_layer* L, int64_t M);
int mid_slice_chunks(const gptq_layer* L, int64_t M);
int tiled_slice_chunks(const gptq_layer* L, int64_t M);
size_t ws_mid_part_bytes(const gptq_layer* L, int64_t M);
// Split-K partial sums of the tiled family ([KS][M][N] fp32 after the x copy and row exponents).
size_t ws_tiled_part_bytes(const gptq_layer* L, int64_t M);

// y[m, n] = round(sum over s = 0 .. KS-1 in order of part[s][m][n] + bias[n]) for rows*N outputs
// (N a multiple of 4): the second launch of every split-K call (mid.hip).
hipError_t launch_part_reduce(const float* part, uint16_t* y, int64_t rows, int N, int KS, const void* bias,
                              int bias_kind, int x_bf16, hipStream_t s);

// The device read floor (read_floor.hip): reads `bytes` at p once.
hipError_t launch_read_floor(const void* p, size_t bytes, uint32_t* sink, hipStream_t s);

// Family launchers.  All assume the call was validated.
hipError_t launch_skinny(const GemmCall& c);
hipError_t launch_mid(const GemmCall& c);
hipError_t launch_tiled(const GemmCall& c);
// x -> workspace copy in the sorted input order (identity without act-order); with to_f16, a bf16
// x becomes fp16 after a per-row power-of-two scaling whose exponents follow the copy.
hipError_t launch_prep(const GemmCall& c, bool to_f16);

constexpr int64_t kSkinnyMaxM = 64;

// Segment -> group map of a layer (layout.h, group_of_segment): d = segments per group, 2^30 for
// one group.  A segment is a 128-input chunk (seg_steps 4) or a 32-input step (seg_steps 1); a layer
// has fewer than 2^15 segments, so the magic-number division is exact.
inline void segment_divisor(const gptq_layer* L, uint32_t* magic, int* shift) {
  const int64_t d = L->group_size == -1 ? (int64_t(1) << 30) : L->gs_eff / (32 * L->seg_steps);
  *shift = segment_shift(d);
  *magic = segment_magic(d);
}

}  // namespace gq
