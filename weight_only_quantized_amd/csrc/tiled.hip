// Tiled family (M > 64): an MFMA-bound GEMM with the weight operand dequantised in registers.
//
// "Formats and kernels: FP8, INT8, INT4, Marlin, Machete" (the batch-size crossover and the
// software-pipelining discussion) places large M on the matrix cores: the packed weight must stay
// packed from HBM to the registers that feed the matrix instruction, conversion runs on the
// vector ALU in the matrix core's slack, and loads of tile k+1 are in flight while tile k
// multiplies; group scales act inside the K reduction.  Design on gfx950:
//   * workgroup tile BM x BN = (16 WM) x (64 WN) with four waves side by side along N, each wave
//     owning WM x WN tiles of 16 x 16 (v_mfma_f32_16x16x32);
//   * the x tile of one 128-input chunk is staged global -> registers -> LDS (double-buffered,
//     rows padded by 16 bytes so a 16-row A-operand read hits distinct banks); each wave reads its
//     A operands from LDS;
//   * each wave loads its own packed weight units straight into registers (one 16-byte load per
//     unit per lane, 4-bit) and builds exact B operands (dequant.h) -- nothing dequantised is ever
//     written to LDS or HBM;
//   * for bf16 activations the operand carries a constant bias of 144; its correction
//     -144 * sum_k x comes from a per-row, per-segment table computed once per call by
//     prep_kernel (the call's workspace) and enters as the MFMA starting accumulator; fp16
//     operands are exact and need no table; the group scale multiplies each segment's fp32
//     partial;
//   * workgroup ids are remapped so that the 32 workgroups resident on one XCD share an x row
//     block (L2) while all XCDs walk the same weight column blocks (MALL).
#include <hip/hip_runtime.h>

#include "dequant.h"
#include "internal.h"

namespace gq {

static inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }
static inline int seg_k(const gptq_layer* L) { return 32 * L->seg_steps; }

size_t ws_xsorted_bytes(const gptq_layer* L, int64_t M) { return align256((size_t)M * L->Kp * 2); }
size_t ws_nsb_bytes(const gptq_layer* L, int64_t M) { return align256((size_t)M * (L->Kp / seg_k(L)) * 4); }

// ---------------------------------------------------------------------------------------------
// prep: xs[m, j] = x[m, perm[j]] (0 past K) and/or nsb[m, s] = -bias * sum_{j in segment s} x.
// One thread per 8 sorted inputs of one row.
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) prep_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
                                                   uint16_t* __restrict__ xs, float* __restrict__ nsb,
                                                   int M, int K, int Kp, int segk, int bf16, float neg_bias) {
  const int j0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (j0 >= Kp) return;  // Kp is a multiple of 128: whole 16-thread groups leave together
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
  const uint16_t* xr = x + (int64_t)m * K;
  uint16_t v[8];
  if (perm) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + e;
      v[e] = j < K ? xr[perm[j]] : (uint16_t)0;
    }
  } else if (j0 < K) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(xr + j0);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[2 * e] = (uint16_t)(w[e] & 0xFFFF); v[2 * e + 1] = (uint16_t)(w[e] >> 16); }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0;
  }
  if (xs) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (uint32_t)v[2 * e] | ((uint32_t)v[2 * e + 1] << 16);
    *reinterpret_cast<u32x4*>(xs + (int64_t)m * Kp + j0) = w;
  }
  if (nsb) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      s += bf16 ? __builtin_bit_cast(float, (uint32_t)v[e] << 16) : (float)__builtin_bit_cast(_Float16, v[e]);
    const int per = segk / 8;  // threads per segment: 16 or 4, aligned groups of lanes
    for (int o = per / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if ((threadIdx.x & (per - 1)) == 0) nsb[(int64_t)m * (Kp / segk) + j0 / segk] = neg_bias * s;
  }
  }
}

static float bias_of(int bits, int bf16) { return (bf16 && bits <= 4) ? 144.f : 0.f; }
bool needs_nsb(const gptq_layer* L, int x_bf16) { return bias_of(L->bits, x_bf16) != 0.f; }

hipError_t launch_prep(const GemmCall& c, bool write_xsorted, bool write_nsb) {
  const gptq_layer* L = c.L;
  uint16_t* xs = nullptr;
  float* nsb = nullptr;
  uint8_t* base = reinterpret_cast<uint8_t*>(c.ws);
  if (write_xsorted) { xs = reinterpret_cast<uint16_t*>(base); base += ws_xsorted_bytes(L, c.M); }
  if (write_nsb) nsb = reinterpret_cast<float*>(base);
  dim3 grid((unsigned)((L->Kp / 8 + 255) / 256), (unsigned)(c.M < 65535 ? c.M : 65535));
  hipLaunchKernelGGL(prep_kernel, grid, dim3(256), 0, c.stream, reinterpret_cast<const uint16_t*>(c.x),
                     write_xsorted ? L->perm : nullptr, xs, nsb, (int)c.M, L->K, L->Kp, seg_k(L), c.x_bf16,
                     -bias_of(L->bits, c.x_bf16));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// The tiled GEMM.
// ---------------------------------------------------------------------------------------------
struct TiledArgs {
  const uint32_t* wq;
  const uint32_t* meta;     // per (tile, group, column): scale bits | stored zero << 16
  const uint32_t* scale32;  // f32 scale bits (scale_kind == 2 only)
  const uint16_t* x;     // [M, ld] sorted-order activations
  const float* nsb;      // [M, Kp / segk]
  uint16_t* y;
  int64_t ld;
  int M, K, N, KC, CT, G, gs_eff, scale_kind, MB, NB;
};

constexpr int kLdsRow = kChunkK + 8;   // halves per LDS row of the x tile (16-byte pad)

template <int BITS, int XT, int WM, int WN, int SEG>
__global__ void __launch_bounds__(256) tiled_kernel(const TiledArgs a) {
  constexpr int BM = 16 * WM;
  constexpr int NSEG = 4 / SEG;
  constexpr int PARTS = BITS == 8 ? 2 : 1;
  constexpr int PW = BITS == 8 ? 4 : BITS;
  constexpr int A_LOADS = BM * (kChunkK * 2 / 16) / 256;   // 16-byte loads per thread per chunk
  static_assert(A_LOADS * 256 == BM * 16, "tile rows must be a multiple of 16");
  __shared__ __attribute__((aligned(16))) uint16_t xs_lds[2][BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) float nsb_lds[2][NSEG][BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, q = lane >> 4;

  // XCD-aware remap of the linear workgroup id (see the file comment).
  const int total = a.MB * a.NB;
  int lid = blockIdx.x;
  if ((total & 7) == 0) lid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int mb = lid / a.NB, nb = lid % a.NB;
  const int m0 = mb * BM;
  const int ct0 = nb * (4 * WN) + wave * WN;

  bool tvalid[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) tvalid[j] = ct0 + j < a.CT;

  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t unit_w = (int64_t)64 * BITS;
  const int nseg_row = a.KC * NSEG;

  struct Stage {
    u32x4 xa[A_LOADS];
    float nsb[2];
    uint32_t w[WN][BITS];
    uint32_t rec[WN][NSEG];     // metadata records (raw: converted at use)
    uint32_t s32[WN][NSEG];
  };

  auto gload = [&](int kc, Stage& st) {
#pragma unroll
    for (int p = 0; p < A_LOADS; ++p) {
      const int idx = p * 256 + tid;           // 16 threads per row, 16-byte pieces
      const int r = idx >> 4, c16 = idx & 15;
      const int m = m0 + r;
      const int k = kc * kChunkK + c16 * 8;
      if (m < a.M && k < a.K)
        st.xa[p] = *reinterpret_cast<const u32x4*>(a.x + (int64_t)m * a.ld + k);
      else
        st.xa[p] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = p * 256 + tid;
      st.nsb[p] = 0.f;
      if (Bias<BITS, XT>::any && idx < BM * NSEG) {
        const int r = idx % BM, s = idx / BM;
        const int m = m0 + r;
        if (m < a.M) st.nsb[p] = a.nsb[(int64_t)m * nseg_row + kc * NSEG + s];
      }
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int ctj = min(ct0 + j, a.CT - 1);     // past-the-end tiles read the last tile, unused
      const uint32_t* u = a.wq + ((int64_t)ctj * a.KC + kc) * unit_w;
#pragma unroll
      for (int p = 0; p < PARTS; ++p) {
        const uint32_t* src = u + p * 64 * PW + lane * PW;
        if constexpr (PW == 4) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(src);
          st.w[j][4 * p + 0] = v[0]; st.w[j][4 * p + 1] = v[1]; st.w[j][4 * p + 2] = v[2]; st.w[j][4 * p + 3] = v[3];
        } else {
#pragma unroll
          for (int e = 0; e < PW; ++e) st.w[j][e] = src[e];
        }
      }
#pragma unroll
      for (int s = 0; s < NSEG; ++s) {
        const int g = min((kc * kChunkK + s * 32 * SEG) / a.gs_eff, a.G - 1);
        const int64_t mi = ((int64_t)ctj * a.G + g) * 16 + col;
        st.rec[j][s] = a.meta[mi];
        if (a.scale_kind == 2) st.s32[j][s] = a.scale32[mi];
      }
    }
  };

  auto lstore = [&](int buf, const Stage& st) {
#pragma unroll
    for (int p = 0; p < A_LOADS; ++p) {
      const int idx = p * 256 + tid;
      const int r = idx >> 4, c16 = idx & 15;
      *reinterpret_cast<u32x4*>(&xs_lds[buf][r * kLdsRow + c16 * 8]) = st.xa[p];
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int idx = p * 256 + tid;
      if (idx < BM * NSEG) nsb_lds[buf][idx / BM][idx % BM] = st.nsb[p];
    }
  };

  auto compute = [&](int buf, const Stage& st) {
    u32x4 b[WN][4];
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        b[j][t] = build_b<BITS, XT>(st.w[j], t, zero_term<BITS, XT>(stored_zero_of(st.rec[j][t / SEG])));
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      u32x4 af[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        af[t] = *reinterpret_cast<const u32x4*>(&xs_lds[buf][(i * 16 + col) * kLdsRow + 32 * t + 8 * q]);
      f32x4 c0[NSEG];
#pragma unroll
      for (int s = 0; s < NSEG; ++s)
        c0[s] = Bias<BITS, XT>::any ? *reinterpret_cast<const f32x4*>(&nsb_lds[buf][s][i * 16 + 4 * q])
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int s = 0; s < NSEG; ++s) {
          f32x4 tmp = c0[s];
#pragma unroll
          for (int t = s * SEG; t < (s + 1) * SEG; ++t) tmp = mfma16<XT>(af[t], b[j][t], tmp);
          acc[i][j] += scale_of(st.rec[j][s], st.s32[j][s], a.scale_kind) * tmp;
        }
    }
  };

  Stage cur, nxt;
  gload(0, cur);
  lstore(0, cur);
  __syncthreads();
  for (int kc = 0; kc < a.KC; ++kc) {
    const int buf = kc & 1;
    const bool more = kc + 1 < a.KC;
    if (more) gload(kc + 1, nxt);
    compute(buf, cur);
    if (more) lstore(buf ^ 1, nxt);
    __syncthreads();
    cur = nxt;
  }

#pragma unroll
  for (int j = 0; j < WN; ++j) {
    if (!tvalid[j]) continue;
    const int n = (ct0 + j) * 16 + col;
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + i * 16 + 4 * q + r;
        if (m < a.M) a.y[(int64_t)m * a.N + n] = to_out<XT>(acc[i][j][r]);
      }
  }
}

template <int BITS, int XT, int WM, int WN>
static hipError_t run_tiled(const TiledArgs& a0, int seg, hipStream_t s) {
  TiledArgs a = a0;
  a.MB = (a.M + 16 * WM - 1) / (16 * WM);
  a.NB = (a.CT + 4 * WN - 1) / (4 * WN);
  const unsigned blocks = (unsigned)(a.MB * a.NB);
  if (seg == 4)
    hipLaunchKernelGGL((tiled_kernel<BITS, XT, WM, WN, 4>), dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((tiled_kernel<BITS, XT, WM, WN, 1>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int XT>
static hipError_t run_tiled_bits(const TiledArgs& a, int bits, int seg, hipStream_t s) {
  switch (bits) {
    case 2: return run_tiled<2, XT, 8, 4>(a, seg, s);
    case 3: return run_tiled<3, XT, 8, 4>(a, seg, s);
    case 4: return run_tiled<4, XT, 8, 4>(a, seg, s);
    default: return run_tiled<8, XT, 8, 4>(a, seg, s);
  }
}

hipError_t launch_tiled(const GemmCall& c) {
  const gptq_layer* L = c.L;
  const bool nsb = needs_nsb(L, c.x_bf16);
  if (L->has_perm || nsb) {
    hipError_t e = launch_prep(c, L->has_perm != 0, nsb);
    if (e != hipSuccess) return e;
  }
  TiledArgs a;
  uint8_t* base = reinterpret_cast<uint8_t*>(c.ws);
  if (L->has_perm) {
    a.x = reinterpret_cast<const uint16_t*>(base);
    a.ld = L->Kp;
    base += ws_xsorted_bytes(L, c.M);
  } else {
    a.x = reinterpret_cast<const uint16_t*>(c.x);
    a.ld = L->K;
  }
  a.nsb = nsb ? reinterpret_cast<const float*>(base) : nullptr;
  a.wq = L->wq;
  a.meta = L->meta;
  a.scale32 = L->scale32;
  a.y = reinterpret_cast<uint16_t*>(c.y);
  a.M = (int)c.M; a.K = L->K; a.N = L->N; a.KC = L->KC; a.CT = L->CT; a.G = L->G;
  a.gs_eff = L->gs_eff;
  a.scale_kind = L->scales_dtype;
  a.MB = a.NB = 0;
  return c.x_bf16 ? run_tiled_bits<1>(a, L->bits, L->seg_steps, c.stream)
                  : run_tiled_bits<0>(a, L->bits, L->seg_steps, c.stream);
}

}  // namespace gq
