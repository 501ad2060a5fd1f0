// Load-time repack: checkpoint tensors -> runtime layout (see layout.h).
//
// Reads the AutoGPTQ pack of "GPTQ packed checkpoint (safetensors / torch)", section "Reader":
// codes run along the input dimension, low bits first, 32/bits per word for 2/4/8 bits; 3-bit
// codes form one 96-bit little-endian stream per 32 codes over three consecutive rows (the
// "10 / split / 10" layout).  qzeros uses the same rule along the output dimension.  Inputs are
// visited in the load-time sorted order ("39. Quantized checkpoints ...", "The format").  The
// same kernels read the other accepted encodings of the same W (RepackSource): GPTQ v2 zeros,
// GPTQ_P planar words (every width 2..8 into the runtime layout of its own width) and AutoAWQ GEMM.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace gq {

// Code of input k, output n from a row-packed int32 array `w` with `ld` words per row.
__device__ __forceinline__ uint32_t packed_field(const uint32_t* __restrict__ w, int64_t ld, int bits,
                                                 int64_t k, int64_t n) {
  if (bits == 3) {
    const int64_t blk = k >> 5;
    const int bit = 3 * (int)(k & 31);
    const int64_t row = 3 * blk + (bit >> 5);
    const int sh = bit & 31;
    uint32_t v = w[row * ld + n] >> sh;
    if (sh > 29) v |= w[(row + 1) * ld + n] << (32 - sh);
    return v & 7u;
  }
  const int pack = 32 / bits;
  const uint32_t v = w[(k / pack) * ld + n];
  return (v >> (bits * (int)(k % pack))) & ((1u << bits) - 1u);
}

// AutoAWQ GEMM pack ("39. Quantized checkpoints ...", section "AWQ"): row r, output n is the
// 4-bit field at bit 4 * pos(n % 8) of word n / 8, where pos inverts the order 0 2 4 6 1 3 5 7:
// pos(c) = 4 (c & 1) + c / 2.
__device__ __forceinline__ uint32_t awq_field(const uint32_t* __restrict__ w, int64_t ld, int64_t r, int64_t n) {
  const int c = (int)(n & 7);
  const int pos = ((c & 1) << 2) | (c >> 1);
  return (w[r * ld + (n >> 3)] >> (4 * pos)) & 0xFu;
}

// GPTQ_P planar words ("Kernel Backends Reference", section "Planar packing"): the 32 codes of
// block k / 32 take rows (k / 32) * bits .. + bits - 1, one run of w rows per plane (widths low
// to high); plane p's field of code j = k % 32 sits at bit w * (j % (32 / w)) of the run's row
// j / (32 / w) and holds code bits [low_p, low_p + w).  `at(row)` reads one word of the run.
template <typename At>
__device__ __forceinline__ uint32_t planar_field(At at, int bits, int j) {
  int w[3], np = 0;
  if (bits == 3) { w[0] = 2; w[1] = 1; np = 2; }
  else if (bits <= 4 || bits == 8) { w[0] = bits; np = 1; }
  else { w[0] = 4; w[1] = bits == 5 ? 1 : 2; w[2] = 1; np = bits == 7 ? 3 : 2; }
  uint32_t code = 0;
  int row = 0, low = 0;
  for (int p = 0; p < np; ++p) {
    const int per = 32 / w[p];
    code |= ((at(row + j / per) >> (w[p] * (j % per))) & ((1u << w[p]) - 1u)) << low;
    row += w[p];
    low += w[p];
  }
  return code;
}

// Same rule along the row (qzeros: group row g, output column n).
__device__ __forceinline__ uint32_t packed_field_cols(const uint32_t* __restrict__ w, int64_t ld, int bits,
                                                      int64_t g, int64_t n) {
  if (bits == 3) {
    const int64_t blk = n >> 5;
    const int bit = 3 * (int)(n & 31);
    const int64_t col = 3 * blk + (bit >> 5);
    const int sh = bit & 31;
    uint32_t v = w[g * ld + col] >> sh;
    if (sh > 29) v |= w[g * ld + col + 1] << (32 - sh);
    return v & 7u;
  }
  const int pack = 32 / bits;
  const uint32_t v = w[g * ld + n / pack];
  return (v >> (bits * (int)(n % pack))) & ((1u << bits) - 1u);
}

// One thread per (unit, lane): gathers the lane's 32 codes and writes its `bits` words.
__global__ void __launch_bounds__(256) repack_words_kernel(
    const uint32_t* __restrict__ qweight, const int32_t* __restrict__ perm, uint32_t* __restrict__ out,
    int K, int N, int bits, int src_bits, int KC, int64_t n_lanes, int src) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_lanes) return;
  const int lane = (int)(gid & 63);
  const int64_t unit = gid >> 6;
  const int kc = (int)(unit % KC);
  const int64_t ct = unit / KC;
  const int64_t n = ct * kTileN + lane_col(lane);
  uint32_t words[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i = 0; i < 32; ++i) {
    const int ks = kc * kChunkK + code_k_in_chunk(lane, i);
    uint32_t code = 0;
    if (ks < K) {
      const int k = perm[ks];
      if (src == kSrcAwqGemm) {
        code = awq_field(qweight, N / 8, k, n);
      } else if (src == kSrcGptqPlanar) {
        const int64_t r0 = (int64_t)(k >> 5) * src_bits;
        code = planar_field([&](int r) { return qweight[(r0 + r) * N + n]; }, src_bits, k & 31);
      } else {
        code = packed_field(qweight, N, src_bits, k, n);
      }
    }
    Piece p[kMaxPieces];
    const int np = code_pieces(bits, i, p);
    for (int q = 0; q < np; ++q) {
      const uint32_t part = (code >> p[q].cbit) & ((1u << p[q].nb) - 1u);
      words[p[q].word] |= part << p[q].bit;
    }
  }
  uint32_t* u = out + unit * unit_words(bits);
  for (int w = 0; w < bits; ++w) u[unit_word_offset(bits, lane, w)] = words[w];
}

// One thread per (tile, group, column-in-tile): scale bits and zero - 1 (mod 2^16; layout.h).
__global__ void __launch_bounds__(256) repack_meta_kernel(
    const uint32_t* __restrict__ qzeros, const void* __restrict__ scales, int scale_bytes,
    uint32_t* __restrict__ meta, uint32_t* __restrict__ scale32, int N, int G, int bits, int64_t total, int src) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int j = (int)(gid & 15);
  const int64_t cg = gid >> 4;          // ct * G + g
  const int g = (int)(cg % G);
  const int64_t ct = cg / G;
  const int64_t n = ct * kTileN + j;
  const int64_t zld = (int64_t)N / 32 * bits;
  uint32_t stored;
  if (src == kSrcAwqGemm) {
    stored = awq_field(qzeros, N / 8, g, n);
  } else if (src == kSrcGptqPlanar) {
    const int64_t c0 = (n >> 5) * bits;
    stored = planar_field([&](int c) { return qzeros[g * zld + c0 + c]; }, bits, (int)(n & 31));
  } else {
    stored = packed_field_cols(qzeros, zld, bits, g, n);
  }
  // v1 layers store zero - 1 already; v2 and AWQ store the zero itself
  const uint32_t z = (src == kSrcGptq || src == kSrcGptqPlanar) ? stored : ((stored - 1u) & 0xFFFFu);
  if (scale_bytes == 4) {
    meta[gid] = z << 16;
    scale32[gid] = reinterpret_cast<const uint32_t*>(scales)[(int64_t)g * N + n];
  } else {
    meta[gid] = (uint32_t)reinterpret_cast<const uint16_t*>(scales)[(int64_t)g * N + n] | (z << 16);
  }
}

hipError_t launch_repack(const gptq_layer* L, const int32_t* qweight, const int32_t* qzeros,
                         const void* scales, RepackSource src, hipStream_t s) {
  const int64_t n_lanes = (int64_t)L->CT * L->KC * kLanes;
  const int64_t blocks = (n_lanes + 255) / 256;
  hipLaunchKernelGGL(repack_words_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(qweight), L->perm, L->wq, L->K, L->N, L->bits,
                     L->ckpt_bits, L->KC, n_lanes, (int)src);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = (int64_t)L->CT * L->G * kTileN;
  hipLaunchKernelGGL(repack_meta_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(qzeros), scales, L->scales_dtype == GPTQ_F32 ? 4 : 2,
                     L->meta, L->scale32, L->N, L->G, L->ckpt_bits, total, (int)src);
  return hipGetLastError();
}

}  // namespace gq
