// Mid family (small M whose x does not fit one workgroup's LDS whole, up to M = 64): a
// memory-bound streaming kernel with split K.
//
// Same method and operand construction as the skinny family (dequant.h; "Formats and kernels:
// FP8, INT8, INT4, Marlin, Machete", the tiny-M tile and split-K discussion): the packed weights
// are read once, from HBM straight into the registers that build exact B operands.  What changes
// with M in the tens is the activation side: loading x per wave from L2 would move several times
// the weight bytes, so here
//   * a workgroup owns BN = 16 WN NW output columns and one slice of the sorted K (KS slices in
//     all); it copies x[0:M, its slice] into LDS once (buffer_load ... lds, rows XOR-swizzled as
//     in the tiled family), and every wave reads its A operands from there;
//   * each wave streams the packed units of its WN column tiles through a register ring DEPTH
//     (2) chunks deep; every workgroup handles exactly TCH chunks, emitted as straight-line code with
//     unconditional loads (chunk indices clamped; x past K is zero), so each chunk waits only for
//     its own loads -- a loop back-edge or a conditional load would make the compiler wait for
//     every load in flight;
//   * with KS > 1 the workgroups store fp32 partial sums [KS][M][N] to the workspace and a second
//     kernel adds them in slice order and rounds (deterministic, no atomics);
//   * bf16 activations use the biased operand of dequant.h: one extra MFMA per step against the
//     constant -144 operand seeds each segment with -144 * sum_k x.
#pragma once
#include <hip/hip_runtime.h>

#include "bufmem.h"
#include "dequant.h"
#include "internal.h"
#include "plans.h"

namespace gq {

struct MidArgs {
  const uint32_t* wq;
  const uint32_t* meta;
  const uint32_t* scale32;
  const uint16_t* x;      // [M, ld] activations in sorted input order
  float* part;            // [KS, M, N] fp32 partial sums (KS > 1)
  uint16_t* y;            // [M, N] (KS == 1)
  int ld;
  int M, K, N, KC, CT, G, scale_kind;
  uint32_t gmagic;       // segment -> group map (segment_divisor)
  int gshift;
  int cpw;                // chunks per K slice (TCH)
  const void* bias;       // [N] in the scales' dtype (scale_kind), or NULL; added when KS == 1
};

// Group of segment `si` (a chunk, or a 32-input step); wave-uniform.
__device__ __forceinline__ int mid_segment_group(int si, uint32_t gmagic, int gshift, int G) {
  return group_of_segment(si, gmagic, gshift, G);
}

// F32S: float32 scales in a parallel array (one more load per chunk); otherwise none is issued.
// XMAP: 0 = workgroups in launch order; 1 / 2 = renumbered so that each XCD (workgroup i runs on
// XCD i mod 8) takes one contiguous run of (column block, slice) pairs, column-block-major (1: an
// XCD walks the slices of consecutive column blocks, i.e. contiguous weight bytes) or slice-major
// (2: an XCD walks the column blocks of one slice, sharing its x slice in L2).  Measured on MI355X
// (8192 x 28672 bf16, 8-chunk slices, with the reduction; us): M = 8 30.9 / 31.1 / 30.4, M = 16
// 33.4 / 32.5 / 32.6; deeper weight rings (4, 8 chunks) 1-3 us slower in every numbering.
template <int BITS, int XT, int MT, int WN, int NW, int SEG, int DEPTH, int TCH, int F32S, int XMAP = 2>
__global__ void __launch_bounds__(64 * NW) mid_kernel(const MidArgs a) {
  constexpr int BMR = 16 * MT;                  // rows held in LDS (rows >= M are zero)
  constexpr int NSEG = 4 / SEG;
  constexpr int PARTS = BITS > 4 ? 2 : 1;      // loads per lane per unit (load_unit)
  constexpr uint32_t UNIT_BYTES = 256u * BITS;
  constexpr bool BIAS = Bias<BITS, XT>::any;
  extern __shared__ __attribute__((aligned(1024))) uint8_t slab[];   // [chunk][row][16 pieces]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, q = lane >> 4;
  int nb = blockIdx.x, ks = blockIdx.y;
  if constexpr (XMAP != 0) {
    const int nbx = gridDim.x, nks = gridDim.y, total = nbx * nks;
    const int lin = blockIdx.x + blockIdx.y * nbx;
    const int x = lin & 7, l = lin >> 3, q = total >> 3, r = total & 7;
    const int id = x * q + (x < r ? x : r) + l;
    if constexpr (XMAP == 1) { nb = id / nks; ks = id - nb * nks; }
    else { ks = id / nbx; nb = id - ks * nbx; }
  }
  const int k0 = ks * TCH;
  const int ct0 = nb * (NW * WN) + wave * WN;

  // ---- buffer resources of the wave's column tiles --------------------------------------------
  rsrc_t rw[WN], rm[WN], rs[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int64_t ctj = min(ct0 + j, a.CT - 1);   // past-the-end tiles alias the last tile, unused
    rw[j] = make_rsrc(a.wq + ctj * a.KC * (64 * BITS), (uint32_t)a.KC * UNIT_BYTES);
    rm[j] = make_rsrc(a.meta + ctj * a.G * 16, (uint32_t)a.G * 64u);
    rs[j] = make_rsrc(a.scale32 ? a.scale32 + ctj * a.G * 16 : a.meta, a.scale32 ? (uint32_t)a.G * 64u : 0u);
  }
  const uint32_t voff_w = unit_voff0<BITS>(lane), voff_w1 = unit_voff1<BITS>(lane);
  const uint32_t voff_m = (uint32_t)col * 4u;
  struct WChunk {
    uint32_t w[WN][BITS];
    uint32_t rec[WN][NSEG];
    uint32_t s32[WN][NSEG];
  };
  auto load_w = [&](int kc, WChunk& c) {
#pragma unroll
    for (int j = 0; j < WN; ++j)
      load_unit<BITS, kAuxStream>(rw[j], voff_w, voff_w1, (uint32_t)kc * UNIT_BYTES, c.w[j]);
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const int g = mid_segment_group(SEG == 4 ? kc : kc * 4 + s, a.gmagic, a.gshift, a.G);
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        c.rec[j][s] = load_b32(rm[j], voff_m, (uint32_t)g * 64u);
        if constexpr (F32S) c.s32[j][s] = load_b32(rs[j], voff_m, (uint32_t)g * 64u);
        else c.s32[j][s] = 0u;
      }
    }
  };

  // ---- weight ring first (HBM latency overlaps the x copy) --------------------------------
  WChunk ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load_w(min(k0 + d, a.KC - 1), ring[d]);

  // ---- x slice -> LDS: slot s of chunk c, row r holds piece (s ^ (r & 15)) --------------------
  {
    const rsrc_t rx = make_rsrc(a.x, (uint32_t)((int64_t)a.M * a.ld * 2));
    constexpr int NINST = TCH * BMR / 4;         // 1 KB DMA instructions (64 slots each)
    static_assert(NINST % NW == 0, "x slice must split evenly over the waves");
#pragma unroll
    for (int u = 0; u < NINST / NW; ++u) {
      const int d = u * NW + wave;
      const int slot = d * 64 + lane;
      const int c = slot / (BMR * 16), rem = slot % (BMR * 16);
      const int r = rem >> 4, pc = (rem & 15) ^ (r & 15);
      const int k = (k0 + c) * kChunkK + pc * 8;
      const uint32_t vo = (r < a.M && k < a.K) ? (uint32_t)(r * a.ld + k) * 2u : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(&slab[d * 1024]), 16, vo, 0u, 0, 0);
    }
  }
  // every wave's share of the copy (and its ring) has landed before any wave reads the slice
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x4 acc[MT][WN];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 nbias;
  nbias[0] = nbias[1] = nbias[2] = nbias[3] = Bias<BITS, XT>::neg2;
  // A operand of row block m, step t, chunk c: row m*16 + col, piece 4t + q
  uint32_t a_off[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) a_off[t] = (uint32_t)(col * 16 + ((4 * t + q) ^ col)) * 16u;

  auto compute = [&](int c, const WChunk& wc) {
    u32x4 b[WN][4];
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        b[j][t] = build_b<BITS, XT>(wc.w[j], t, zero_term<BITS, XT>(zero_of(wc.rec[j][t / SEG])));
    float sc[WN][NSEG];
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int s = 0; s < NSEG; ++s) sc[j][s] = scale_of(wc.rec[j][s], wc.s32[j][s], a.scale_kind);
    const uint8_t* xb = slab + (size_t)c * (BMR * 256);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      u32x4 af[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) af[t] = *reinterpret_cast<const u32x4*>(xb + a_off[t] + m * 4096);
      f32x4 c0[NSEG];
#pragma unroll
      for (int s = 0; s < NSEG; ++s) {
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (BIAS) {
#pragma unroll
          for (int t = s * SEG; t < (s + 1) * SEG; ++t) v = mfma16<XT>(af[t], nbias, v);
        }
        c0[s] = v;
      }
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int s = 0; s < NSEG; ++s) {
          f32x4 tmp = c0[s];
#pragma unroll
          for (int t = s * SEG; t < (s + 1) * SEG; ++t) tmp = mfma16<XT>(af[t], b[j][t], tmp);
          acc[m][j] += sc[j][s] * tmp;
        }
    }
  };

  // ---- chunk c from ring slot c % DEPTH, then refill it with chunk c + DEPTH ---------------
  // (straight-line: the refills past the slice are left out at compile time)
#pragma unroll
  for (int base = 0; base < TCH; base += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      compute(base + d, ring[d]);
      if (base + d + DEPTH < TCH) load_w(min(k0 + base + d + DEPTH, a.KC - 1), ring[d]);
    }
  }

  // ---- store: y directly (one slice) or this slice's fp32 partial ---------------------------
  const bool whole = gridDim.y == 1;
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    if (ct0 + j >= a.CT) continue;
    const int n = (ct0 + j) * 16 + col;
    const float bn = whole ? bias_at(a.bias, a.scale_kind, n) : 0.f;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m * 16 + 4 * q + r;
        if (row >= a.M) continue;
        if (whole) a.y[(int64_t)row * a.N + n] = to_out<XT>(acc[m][j][r] + bn);
        else a.part[((int64_t)ks * a.M + row) * a.N + n] = acc[m][j][r];
      }
  }
}

// (the mid plan: plans.h)
inline int64_t mid_rows_per_pass(const gptq_layer* L) { return mid_rows_per_pass_of(L->seg_steps); }
inline MidPlan mid_plan(const gptq_layer* L, int64_t M) { return mid_plan_of(M, L->KC, L->CT, L->seg_steps); }

template <int BITS, int XT, int MT, int SEG, int TCH, int F32S>
static hipError_t run_mid_cfg(const MidArgs& a, int KS, hipStream_t s) {
  constexpr int DEPTH = 2;
  const int nbk = (a.CT + kMidNW * kMidWN - 1) / (kMidNW * kMidWN);
  const size_t lds = (size_t)TCH * 16 * MT * 256;
  hipLaunchKernelGGL((mid_kernel<BITS, XT, MT, kMidWN, kMidNW, SEG, DEPTH, TCH, F32S>), dim3(nbk, KS),
                     dim3(64 * kMidNW), lds, s, a);
  return hipGetLastError();
}

template <int BITS, int XT, int SEG, int F32S>
static hipError_t run_mid_seg(const MidArgs& a, const MidPlan& p, hipStream_t s) {
  if (p.MT == 1) {
    if (p.cpw == 16) return run_mid_cfg<BITS, XT, 1, SEG, 16, F32S>(a, p.KS, s);
    if (p.cpw == 8) return run_mid_cfg<BITS, XT, 1, SEG, 8, F32S>(a, p.KS, s);
    return run_mid_cfg<BITS, XT, 1, SEG, 4, F32S>(a, p.KS, s);
  }
  if (p.MT == 2) {
    if (p.cpw == 8) return run_mid_cfg<BITS, XT, 2, SEG, 8, F32S>(a, p.KS, s);
    return run_mid_cfg<BITS, XT, 2, SEG, 4, F32S>(a, p.KS, s);
  }
  return run_mid_cfg<BITS, XT, 4, SEG, 4, F32S>(a, p.KS, s);
}

// 32-input segments (four scales per chunk) always run 4-chunk slices of at most two row blocks
// (the launcher splits larger M into passes of 32 rows).
template <int BITS, int XT, int F32S>
static hipError_t run_mid_m(const MidArgs& a, const MidPlan& p, int seg, hipStream_t s) {
  if (seg == 4) return run_mid_seg<BITS, XT, 4, F32S>(a, p, s);
  if (p.MT == 1) return run_mid_cfg<BITS, XT, 1, 1, 4, F32S>(a, p.KS, s);
  return run_mid_cfg<BITS, XT, 2, 1, 4, F32S>(a, p.KS, s);
}

template <int BITS>
hipError_t mid_bits(const MidArgs& a, const MidPlan& p, int x_bf16, int seg, hipStream_t s) {
  if (a.scale_kind == 2) return x_bf16 ? run_mid_m<BITS, 1, 1>(a, p, seg, s) : run_mid_m<BITS, 0, 1>(a, p, seg, s);
  return x_bf16 ? run_mid_m<BITS, 1, 0>(a, p, seg, s) : run_mid_m<BITS, 0, 0>(a, p, seg, s);
}
hipError_t mid_b2(const MidArgs& a, const MidPlan& p, int x_bf16, int seg, hipStream_t s);
hipError_t mid_b3(const MidArgs& a, const MidPlan& p, int x_bf16, int seg, hipStream_t s);
hipError_t mid_b4(const MidArgs& a, const MidPlan& p, int x_bf16, int seg, hipStream_t s);
hipError_t mid_b5(const MidArgs& a, const MidPlan& p, int x_bf16, int seg, hipStream_t s);
hipError_t mid_b6(const MidArgs& a, const MidPlan& p, int x_bf16, int seg, hipStream_t s);
hipError_t mid_b7(const MidArgs& a, const MidPlan& p, int x_bf16, int seg, hipStream_t s);
hipError_t mid_b8(const MidArgs& a, const MidPlan& p, int x_bf16, int seg, hipStream_t s);

}  // namespace gq
