// Tiled family (M > 64): an MFMA-bound GEMM with the weight operand dequantised in registers.
//
// "Formats and kernels: FP8, INT8, INT4, Marlin, Machete" (the batch-size crossover and the
// software-pipelining discussion) places large M on the matrix cores: the packed weight must stay
// packed from HBM to the registers that feed the matrix instruction, conversion runs on the
// vector ALU in the matrix core's slack, and loads of tile k+1 are in flight while tile k
// multiplies; group scales act inside the K reduction.  Design on gfx950:
//   * workgroup tile BM x BN = (16 WM) x (64 WN) with four waves side by side along N, each wave
//     owning WM x WN tiles of 16 x 16 (v_mfma_f32_16x16x32); WM = 8, WN = 2 keeps a wave under
//     256 registers so two workgroups share a CU;
//   * the x tile of one 128-input chunk goes global -> LDS directly (buffer_load ... lds,
//     double-buffered, XOR-swizzled so a 16-row A-operand read hits distinct banks); each wave
//     reads its A operands from LDS;
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

#include "bufmem.h"
#include "dequant.h"
#include "internal.h"
#include "skinny_impl.h"

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
  const float* nsb;      // [M, Kp / segk] (bf16 only)
  uint16_t* y;
  int ld;
  int M, K, N, KC, CT, G, scale_kind, MB, NB;
  int gdiv, gshift;      // segment -> group map (see segment_divisor)
};

// x tile of one chunk in LDS: BM rows x 16 pieces of 16 bytes, no padding, piece c of row r at
// slot r * 16 + (c ^ (r & 15)).  Sixteen lanes reading the same piece of sixteen consecutive
// rows (an A operand) then hit sixteen different 16-byte bank groups.  The tile is filled with
// buffer_load ... lds (lane i of a load writes slot i of its 1 KB destination), so each lane
// simply fetches the global piece that belongs in its slot.
template <int BITS, int XT, int WM, int WN, int SEG>
__global__ void __launch_bounds__(256) tiled_kernel(const TiledArgs a) {
  constexpr int BM = 16 * WM;
  constexpr int NSEG = 4 / SEG;
  constexpr int PARTS = BITS == 8 ? 2 : 1;
  constexpr int PW = BITS == 8 ? 4 : BITS;
  constexpr uint32_t UNIT_BYTES = 256u * BITS;
  constexpr int A_BYTES = BM * 256;            // one chunk of x for the tile
  constexpr int A_INST = BM / 16;              // 1 KB LDS loads per wave per chunk
  constexpr bool BIAS = Bias<BITS, XT>::any;
  __shared__ __attribute__((aligned(1024))) uint8_t xs[2][A_BYTES];
  __shared__ __attribute__((aligned(16))) float nsb_s[2][NSEG][BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, q = lane >> 4;

  // XCD-aware remap of the linear workgroup id (see the file comment).
  const int total = a.MB * a.NB;
  int lid = blockIdx.x;
  if ((total & 7) == 0) lid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int mb = lid / a.NB, nb = lid % a.NB;
  const int m0 = mb * BM;
  const int ct0 = nb * (4 * WN) + wave * WN;

  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- resources and fixed per-lane offsets -------------------------------------------------
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)((int64_t)a.M * a.ld * 2));
  uint32_t voff_a[A_INST];
  int kpiece_a[A_INST];                        // input offset of the lane's piece within a chunk
#pragma unroll
  for (int j = 0; j < A_INST; ++j) {
    const int slot = (wave * A_INST + j) * 64 + lane;
    const int r = slot >> 4, c = (slot & 15) ^ (r & 15);
    kpiece_a[j] = c * 8;
    voff_a[j] = (m0 + r < a.M) ? (uint32_t)((m0 + r) * a.ld + c * 8) * 2u : kOob;
  }
  const bool ktail = (a.K & (kChunkK - 1)) != 0;
  rsrc_t rw[WN], rm[WN], rs[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int64_t ctj = min(ct0 + j, a.CT - 1);   // past-the-end tiles alias the last tile, unused
    rw[j] = make_rsrc(a.wq + ctj * a.KC * (64 * BITS), (uint32_t)a.KC * UNIT_BYTES);
    rm[j] = make_rsrc(a.meta + ctj * a.G * 16, (uint32_t)a.G * 64u);
    rs[j] = make_rsrc(a.scale32 ? a.scale32 + ctj * a.G * 16 : a.meta, a.scale32 ? (uint32_t)a.G * 64u : 0u);
  }
  const uint32_t voff_w = (uint32_t)lane * PW * 4u;
  const uint32_t voff_m = (uint32_t)col * 4u;
  const int nseg_row = a.KC * NSEG;
  const rsrc_t rn = make_rsrc(a.nsb, BIAS ? (uint32_t)((int64_t)a.M * nseg_row * 4) : 0u);
  // A operand reads: row i*16 + col, piece 4t + q  ->  byte (col * 16 + ((4t + q) ^ col)) * 16 + i * 4096
  uint32_t a_off[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) a_off[t] = (uint32_t)(col * 16 + ((4 * t + q) ^ col)) * 16u;

  struct Stage {
    uint32_t w[WN][BITS];
    uint32_t rec[WN][NSEG];
    uint32_t s32[WN][NSEG];
    float nsb[2];
  };

  // x chunk kc -> xs[buf] by LDS DMA; packed units, metadata and bias sums -> registers.
  auto issue = [&](int kc, int buf, Stage& st) {
    const bool tail = ktail && kc == a.KC - 1;
#pragma unroll
    for (int j = 0; j < A_INST; ++j) {
      uint32_t vo = voff_a[j];
      if (tail && kc * kChunkK + kpiece_a[j] >= a.K) vo = kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(&xs[buf][(wave * A_INST + j) * 1024]), 16, vo,
          (uint32_t)kc * 256u, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int p = 0; p < PARTS; ++p)
        load_words<PW, 0>(rw[j], voff_w + p * 1024u, (uint32_t)kc * UNIT_BYTES, &st.w[j][4 * p]);
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const int g = segment_group(SEG == 4 ? kc : kc * 4 + s, a.gdiv, a.gshift, a.G);
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        st.rec[j][s] = load_b32(rm[j], voff_m, (uint32_t)g * 64u);
        st.s32[j][s] = load_b32(rs[j], voff_m, (uint32_t)g * 64u);
      }
    }
    if constexpr (BIAS) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int idx = p * 256 + tid;
        const int r = idx % BM, s = idx / BM;
        const bool ok = idx < BM * NSEG && m0 + r < a.M;
        st.nsb[p] = __builtin_bit_cast(float, load_b32(rn, ok ? (uint32_t)((m0 + r) * nseg_row + kc * NSEG + s) * 4u : kOob, 0u));
      }
    }
  };
  auto store_nsb = [&](int buf, const Stage& st) {
    if constexpr (BIAS) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int idx = p * 256 + tid;
        if (idx < BM * NSEG) nsb_s[buf][idx / BM][idx % BM] = st.nsb[p];
      }
    }
  };

  auto compute = [&](int buf, const Stage& st) {
    u32x4 b[WN][4];
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        b[j][t] = build_b<BITS, XT>(st.w[j], t, zero_term<BITS, XT>(stored_zero_of(st.rec[j][t / SEG])));
    float sc[WN][NSEG];
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int s = 0; s < NSEG; ++s) sc[j][s] = scale_of(st.rec[j][s], st.s32[j][s], a.scale_kind);
    const uint8_t* xb = &xs[buf][0];
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      u32x4 af[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) af[t] = *reinterpret_cast<const u32x4*>(xb + a_off[t] + i * 4096);
      f32x4 c0[NSEG];
#pragma unroll
      for (int s = 0; s < NSEG; ++s)
        c0[s] = BIAS ? *reinterpret_cast<const f32x4*>(&nsb_s[buf][s][i * 16 + 4 * q]) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int s = 0; s < NSEG; ++s) {
          f32x4 tmp = c0[s];
#pragma unroll
          for (int t = s * SEG; t < (s + 1) * SEG; ++t) tmp = mfma16<XT>(af[t], b[j][t], tmp);
          acc[i][j] += sc[j][s] * tmp;
        }
    }
  };

  Stage cur, nxt;
  issue(0, 0, cur);
  __builtin_amdgcn_s_waitcnt(0);
  store_nsb(0, cur);
  __syncthreads();
  for (int kc = 0; kc < a.KC; ++kc) {
    const int buf = kc & 1;
    const bool more = kc + 1 < a.KC;
    if (more) issue(kc + 1, buf ^ 1, nxt);
    compute(buf, cur);
    // the next chunk's x tile, units and sums were issued before this chunk's compute
    __builtin_amdgcn_s_waitcnt(0);
    if (more) store_nsb(buf ^ 1, nxt);
    __syncthreads();
    cur = nxt;
  }

#pragma unroll
  for (int j = 0; j < WN; ++j) {
    if (ct0 + j >= a.CT) continue;
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
    // wave tile 128 x 32 (WG tile 128 x 128): ~250 registers -> two workgroups per CU, measured
    // 1.4-1.6x faster on MI355X than a 128 x 64 wave tile at one workgroup per CU
    case 2: return run_tiled<2, XT, 8, 2>(a, seg, s);
    case 3: return run_tiled<3, XT, 8, 2>(a, seg, s);
    case 4: return run_tiled<4, XT, 8, 2>(a, seg, s);
    default: return run_tiled<8, XT, 8, 2>(a, seg, s);
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
  segment_divisor(L, &a.gdiv, &a.gshift);
  a.scale_kind = L->scales_dtype;
  a.MB = a.NB = 0;
  return c.x_bf16 ? run_tiled_bits<1>(a, L->bits, L->seg_steps, c.stream)
                  : run_tiled_bits<0>(a, L->bits, L->seg_steps, c.stream);
}

}  // namespace gq
