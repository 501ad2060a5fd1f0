// Skinny family (M <= 64): a memory-bound streaming kernel.
//
// "Formats and kernels: FP8, INT8, INT4, Marlin, Machete" (its roofline opening and the tiny-M
// tile discussion) explains why small M is bound by the packed weight stream: every byte of the
// weights must be read once, with every compute unit pulling, and the arithmetic hides in the
// slack.  Design on gfx950:
//   * one wave owns TW column tiles (16 columns each) and a slice of the sorted K chunks; the
//     KSPLIT waves of a workgroup that share column tiles split K between them and meet in LDS at
//     the end (deterministic, no atomics, no workspace);
//   * per 128-input chunk a lane issues one 16-byte load per tile (4-bit) of packed runtime words
//     (layout.h), plus one 16-byte load per 16-row block of x for its MFMA A operand; the next
//     chunk's loads are in flight while the current chunk is dequantised and multiplied;
//   * the dequantised operand never leaves registers (dequant.h): B = code - zero exactly for
//     fp16; for bf16 B = 144 + (code - zero) exactly and one extra MFMA per step against a
//     constant -144 operand yields the correction -144 * sum_k x as the starting accumulator of
//     each segment; after a segment the group scale multiplies the fp32 partial into the output
//     accumulator.
#include <hip/hip_runtime.h>

#include "dequant.h"
#include "internal.h"

namespace gq {

struct SkinnyArgs {
  const uint32_t* wq;
  const void* scales;
  const uint8_t* zeros;
  const uint16_t* x;      // [M, ld] activations in sorted input order
  uint16_t* y;            // [M, N]
  int64_t ld;             // row stride of x in elements
  int M, K, N, KC, CT, G, gs_eff, scale_kind;
};

template <int BITS, int XT, int MT, int TW, int KSPLIT, int SEG>
__global__ void __launch_bounds__(256) skinny_kernel(const SkinnyArgs a) {
  constexpr int CGS = 4 / KSPLIT;               // column groups per workgroup
  constexpr int NSEG = 4 / SEG;                 // fixup segments per chunk
  constexpr int PARTS = BITS == 8 ? 2 : 1;      // 16-byte (or smaller) loads per lane per unit
  constexpr int PW = BITS == 8 ? 4 : BITS;      // words per part
  __shared__ float red[4][MT * TW * 4][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cg = wave / KSPLIT, ks = wave % KSPLIT;
  const int ct0 = (blockIdx.x * CGS + cg) * TW;
  const int cpw = (a.KC + KSPLIT - 1) / KSPLIT;
  const int kc0 = ks * cpw;
  const int kc1 = min(a.KC, kc0 + cpw);
  const int col = lane & 15, q = lane >> 4;

  bool tvalid[TW];
#pragma unroll
  for (int i = 0; i < TW; ++i) tvalid[i] = ct0 + i < a.CT;

  f32x4 acc[MT][TW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < TW; ++i) acc[m][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t unit_w = (int64_t)64 * BITS;
  u32x4 nb;
  nb[0] = nb[1] = nb[2] = nb[3] = Bias<BITS, XT>::neg2;

  // ---- one chunk's loads -------------------------------------------------------------------
  struct Chunk {
    uint32_t w[TW][BITS];
    u32x4 xa[MT][4];
    uint32_t zs[TW][NSEG];
    float sc[TW][NSEG];
  };
  auto load = [&](int kc, Chunk& c) {
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      if (tvalid[i]) {
        const uint32_t* u = a.wq + ((int64_t)(ct0 + i) * a.KC + kc) * unit_w;
#pragma unroll
        for (int p = 0; p < PARTS; ++p) {
          const uint32_t* src = u + p * 64 * PW + lane * PW;
          if constexpr (PW == 4) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(src);
            c.w[i][4 * p + 0] = v[0]; c.w[i][4 * p + 1] = v[1]; c.w[i][4 * p + 2] = v[2]; c.w[i][4 * p + 3] = v[3];
          } else {
#pragma unroll
            for (int j = 0; j < PW; ++j) c.w[i][j] = src[j];
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < BITS; ++j) c.w[i][j] = 0u;
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int row = m * 16 + col;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int k = kc * kChunkK + 32 * t + 8 * q;
        if (row < a.M && k < a.K)
          c.xa[m][t] = *reinterpret_cast<const u32x4*>(a.x + (int64_t)row * a.ld + k);
        else
          c.xa[m][t] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const int g = min((kc * kChunkK + s * 32 * SEG) / a.gs_eff, a.G - 1);
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        if (tvalid[i]) {
          const int64_t mi = ((int64_t)(ct0 + i) * a.G + g) * 16 + col;
          c.zs[i][s] = zero_term<BITS, XT>(a.zeros[mi]);
          c.sc[i][s] = scale_value(a.scales, mi, a.scale_kind);
        } else {
          c.zs[i][s] = 0u;
          c.sc[i][s] = 0.f;
        }
      }
    }
  };

  // ---- one chunk's arithmetic --------------------------------------------------------------
  auto compute = [&](const Chunk& c) {
    f32x4 c0[MT][NSEG];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int s = 0; s < NSEG; ++s) {
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (Bias<BITS, XT>::any) {
#pragma unroll
          for (int t = s * SEG; t < (s + 1) * SEG; ++t) v = mfma16<XT>(c.xa[m][t], nb, v);
        }
        c0[m][s] = v;
      }
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      u32x4 b[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) b[t] = build_b<BITS, XT>(c.w[i], t, c.zs[i][t / SEG]);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < NSEG; ++s) {
          f32x4 tmp = c0[m][s];
#pragma unroll
          for (int t = s * SEG; t < (s + 1) * SEG; ++t) tmp = mfma16<XT>(c.xa[m][t], b[t], tmp);
          acc[m][i] += c.sc[i][s] * tmp;
        }
    }
  };

  if (kc0 < kc1) {
    Chunk cur, nxt;
    load(kc0, cur);
    for (int kc = kc0; kc < kc1; ++kc) {
      if (kc + 1 < kc1) load(kc + 1, nxt);
      compute(cur);
      cur = nxt;
    }
  }

  // ---- reduce the KSPLIT partial sums of each column group, then store ---------------------
  if constexpr (KSPLIT > 1) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][(m * TW + i) * 4 + r][lane] = acc[m][i][r];
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int w2 = 1; w2 < KSPLIT; ++w2)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[m][i][r] += red[wave + w2][(m * TW + i) * 4 + r][lane];
  }
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    if (!tvalid[i]) continue;
    const int n = (ct0 + i) * 16 + col;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m * 16 + 4 * q + r;
        if (row < a.M) a.y[(int64_t)row * a.N + n] = to_out<XT>(acc[m][i][r]);
      }
  }
}

// ------------------------------------------------------------------------------------------------
// Dispatch: tiles per wave grow with M so that x traffic (from L2) stays near the weight traffic.
// ------------------------------------------------------------------------------------------------
template <int BITS, int XT, int MT, int TW, int KSPLIT>
static hipError_t run(const SkinnyArgs& a, int seg, hipStream_t s) {
  constexpr int CGS = 4 / KSPLIT;
  const int blocks = (a.CT + TW * CGS - 1) / (TW * CGS);
  if (seg == 4)
    hipLaunchKernelGGL((skinny_kernel<BITS, XT, MT, TW, KSPLIT, 4>), dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((skinny_kernel<BITS, XT, MT, TW, KSPLIT, 1>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int BITS, int XT>
static hipError_t run_m(const SkinnyArgs& a, int seg, hipStream_t s) {
  if (a.M <= 4) return run<BITS, XT, 1, 1, 4>(a, seg, s);
  if (a.M <= 8) return run<BITS, XT, 1, 2, 4>(a, seg, s);
  if (a.M <= 16) return run<BITS, XT, 1, 2, 4>(a, seg, s);
  if (a.M <= 32) return run<BITS, XT, 2, 2, 4>(a, seg, s);
  return run<BITS, XT, 4, 2, 4>(a, seg, s);
}

template <int XT>
static hipError_t run_bits(const SkinnyArgs& a, int bits, int seg, hipStream_t s) {
  switch (bits) {
    case 2: return run_m<2, XT>(a, seg, s);
    case 3: return run_m<3, XT>(a, seg, s);
    case 4: return run_m<4, XT>(a, seg, s);
    default: return run_m<8, XT>(a, seg, s);
  }
}

hipError_t launch_skinny(const GemmCall& c) {
  const gptq_layer* L = c.L;
  SkinnyArgs a;
  a.wq = L->wq;
  a.scales = L->scales_rt;
  a.zeros = L->zeros_rt;
  a.y = reinterpret_cast<uint16_t*>(c.y);
  a.M = (int)c.M; a.K = L->K; a.N = L->N; a.KC = L->KC; a.CT = L->CT; a.G = L->G;
  a.gs_eff = L->gs_eff;
  a.scale_kind = L->scales_dtype;
  if (L->has_perm) {
    hipError_t e = launch_prep(c, true, false);
    if (e != hipSuccess) return e;
    a.x = reinterpret_cast<const uint16_t*>(c.ws);
    a.ld = L->Kp;
  } else {
    a.x = reinterpret_cast<const uint16_t*>(c.x);
    a.ld = L->K;
  }
  return c.x_bf16 ? run_bits<1>(a, L->bits, L->seg_steps, c.stream)
                  : run_bits<0>(a, L->bits, L->seg_steps, c.stream);
}

}  // namespace gq
