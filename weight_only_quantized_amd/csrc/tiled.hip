// Tiled family (M > 16, or > 32 on long K): an MFMA GEMM with the weight operand dequantised in
// registers, from a table of workgroup tiles, with K split over workgroups when the tiles alone
// would leave compute units idle (tiled_plan).
//
// "Formats and kernels: FP8, INT8, INT4, Marlin, Machete" (the batch-size crossover and the
// software-pipelining discussion) places large M on the matrix cores: the packed weight must stay
// packed from HBM to the registers that feed the matrix instruction, conversion runs on the
// vector ALU in the matrix core's slack, and loads of tile k+1 are in flight while tile k
// multiplies; group scales act inside the K reduction.  Design on gfx950:
//   * workgroup tile BM x BN = (16 WM) x (16 WN NW) with NW waves side by side along N, each
//     wave owning WM x WN tiles of 16 x 16 (v_mfma_f32_16x16x32); the large-M tile is 256 x 256
//     (WM = 16, WN = 2, eight waves, two per SIMD, under 256 registers each);
//   * the x tile of one 128-input chunk goes to LDS (XOR-swizzled so a 16-row A-operand read hits
//     distinct banks): by buffer_load ... lds and a full wait with one chunk in flight, through
//     registers with two (see tiled_kernel); each wave reads its A operands from LDS one 16-row
//     block ahead of the matrix instructions that use them, and applies a block's group scales
//     after the next block's MFMAs are issued;
//   * each wave loads its own packed weight units straight into registers (one 16-byte load per
//     unit per lane, 4-bit) and builds exact B operands (dequant.h) -- nothing dequantised is ever
//     written to LDS or HBM;
//   * the group scale multiplies each segment's fp32 partial; the operands are exact fp16
//     (activation, and code - zero);
//   * bf16 activations are converted to fp16 once per call by prep_kernel, exactly, after an
//     exact power-of-two scaling of each row that puts its largest magnitude in [2^14, 2^15); the
//     row's outputs are multiplied back by the same power of two before rounding to bf16.  (bf16
//     B operands would need the +144 bias of dequant.h, whose eight busy mantissa bits measured
//     about 10% slower on the matrix cores than exact small fp16 integers, plus a correction.)
//   * workgroup ids are remapped so that the 32 workgroups resident on one XCD share an x row
//     block (L2) while all XCDs walk the same weight column blocks (MALL); workgroups sharing a
//     row block walk K in step, so each x chunk is fetched into L2 about once per XCD (a
//     staggered K start per column block measured 2-3 % slower and doubled the fabric reads);
//   * the packed units and metadata of the next chunk are requested before its x tile;
//   * split K for the few-tile calls of the mid-batch range that "Formats and kernels ...", section
//     "Tile tables, and what happens when your shape does not fit", buckets: slice ks of KS runs chunks
//     [ks kcs, (ks + 1) kcs) and writes fp32 partial sums; a second launch adds the slices in
//     order with the bias and rounds once (deterministic, no atomics, no counters to clear).
#include <hip/hip_runtime.h>

#include "bufmem.h"
#include "dequant.h"
#include "internal.h"
#include "plans.h"
#include "skinny_impl.h"

namespace gq {

static inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }
size_t ws_xsorted_bytes(const gptq_layer* L, int64_t M) { return align256((size_t)M * L->Kp * 2); }
size_t ws_rowexp_bytes(int64_t M) { return align256((size_t)M * 4); }
// The tiled kernel reads x in whole 128-input chunks, so it takes a zero-padded copy whenever x
// itself is not in that form: act-order (sorted copy), bf16 (fp16 copy), K not a multiple of 128.
bool tiled_needs_xsorted(const gptq_layer* L, int x_bf16) {
  return L->has_perm || x_bf16 || (L->K % kChunkK) != 0;
}

// ---------------------------------------------------------------------------------------------
// prep: workgroup (m, stripe) handles row m, sorted inputs [stripe * span, (stripe + 1) * span)
// (one stripe of the whole row when a row maximum is needed).  xs[m, j] = x[m, perm[j]] (perm may
// be the identity), 0 for
// K <= j < Kp.  With to_f16 (bf16 input): e_m = ilogb(max_k |x[m, k]|) - 14 (0 for an all-zero or
// non-finite maximum), xs holds fp16(x * 2^-e_m) and rowexp[m] = e_m.  The conversion is exact
// except for magnitudes below 2^-17 after scaling (more than 2^31 below the row maximum), which
// land on fp16's subnormal grid.  Without to_f16 the 16-bit values are copied unchanged.
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) prep_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
                                                   uint16_t* __restrict__ xs, int32_t* __restrict__ rowexp, int M,
                                                   int K, int Kp, int to_f16, int span) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int m = blockIdx.x; m < M; m += gridDim.x) {
    const uint16_t* xr = x + (int64_t)m * K;
    int e = 0;
    if (to_f16) {
      float mx = 0.f;
      for (int k = tid * 8; k < K; k += 2048) {   // K is a multiple of 32
        const u32x4 w = *reinterpret_cast<const u32x4*>(xr + k);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          mx = fmaxf(mx, fabsf(__builtin_bit_cast(float, w[q] << 16)));
          mx = fmaxf(mx, fabsf(__builtin_bit_cast(float, w[q] & 0xFFFF0000u)));
        }
      }
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      if (lane == 0) red[wave] = mx;
      __syncthreads();
      mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      __syncthreads();
      if (mx > 0.f && mx <= 3.4028235e38f) e = ilogbf(mx) - 14;
      if (tid == 0) rowexp[m] = e;
    }
    const int jend = min(Kp, (int)blockIdx.y * span + span);
    for (int j0 = (int)blockIdx.y * span + tid * 8; j0 < jend; j0 += 2048) {
      uint16_t v[8];
      if (perm) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = j0 + q;
          v[q] = j < K ? xr[perm[j]] : (uint16_t)0;
        }
      } else if (j0 < K) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(xr + j0);
#pragma unroll
        for (int q = 0; q < 4; ++q) { v[2 * q] = (uint16_t)(w[q] & 0xFFFF); v[2 * q + 1] = (uint16_t)(w[q] >> 16); }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = 0;
      }
      if (to_f16) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float f = ldexpf(__builtin_bit_cast(float, (uint32_t)v[q] << 16), -e);
          v[q] = __builtin_bit_cast(uint16_t, (_Float16)f);
        }
      }
      u32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = (uint32_t)v[2 * q] | ((uint32_t)v[2 * q + 1] << 16);
      *reinterpret_cast<u32x4*>(xs + (int64_t)m * Kp + j0) = w;
    }
  }
}

// prep for bf16 activations without a permutation, rows of at most 2048 * PR inputs: workgroup m
// reads its row once into registers (PR pieces of 8 per thread, all loads in flight together),
// reduces the row maximum, and writes the rescaled fp16 copy from the registers -- the same
// values as prep_kernel with to_f16, in one pass over x instead of two.
template <int PR>
__global__ void __launch_bounds__(256) prep_f16_row_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ xs,
                                                           int32_t* __restrict__ rowexp, int M, int K, int Kp) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int m = blockIdx.x; m < M; m += gridDim.x) {
    const uint16_t* xr = x + (int64_t)m * K;
    u32x4 v[PR];
#pragma unroll
    for (int r = 0; r < PR; ++r) {
      const int j0 = tid * 8 + r * 2048;
      v[r] = j0 < K ? *reinterpret_cast<const u32x4*>(xr + j0) : u32x4{0u, 0u, 0u, 0u};   // K % 8 == 0
    }
    float mx = 0.f;
#pragma unroll
    for (int r = 0; r < PR; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mx = fmaxf(mx, fabsf(__builtin_bit_cast(float, v[r][q] << 16)));
        mx = fmaxf(mx, fabsf(__builtin_bit_cast(float, v[r][q] & 0xFFFF0000u)));
      }
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const int e = (mx > 0.f && mx <= 3.4028235e38f) ? ilogbf(mx) - 14 : 0;
    if (tid == 0) rowexp[m] = e;
#pragma unroll
    for (int r = 0; r < PR; ++r) {
      const int j0 = tid * 8 + r * 2048;
      if (j0 < Kp) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = ldexpf(__builtin_bit_cast(float, v[r][q] << 16), -e);
          const float hi = ldexpf(__builtin_bit_cast(float, v[r][q] & 0xFFFF0000u), -e);
          w[q] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
        }
        *reinterpret_cast<u32x4*>(xs + (int64_t)m * Kp + j0) = w;
      }
    }
  }
}

// prep for act-order layers that carry the 16-bit inverse permutation (Kp <= 8192), copied
// unchanged: workgroup (m, stripe) reads 2048 consecutive inputs of row m and their sorted
// positions (both coalesced, in one round of loads) and stores each value at its position, where
// the gather by the permutation waits for the permutation's loads before issuing the values'.
// The sorted positions K .. Kp - 1 (the padding of the last chunk) get zeros.  Used up to 32 rows
// (MI355X, 8192 x 8192, whole calls: M = 8 / 17 / 32 0.5 / 0.15 / 0.3-0.7 us faster than with the
// gather; at M = 64 / 128 / 1024 the 2-byte scattered stores measured 0.4 / 0-1.1 / 4.5 us slower).
__global__ void __launch_bounds__(256) prep_scatter_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ iperm,
                                                           uint16_t* __restrict__ xs, int M, int K, int Kp) {
  const int k0 = (int)blockIdx.y * 2048 + (int)threadIdx.x * 8;   // K and Kp are multiples of 32
  for (int m = blockIdx.x; m < M; m += gridDim.x) {
    uint16_t* xr = xs + (int64_t)m * Kp;
    if (k0 < K) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(x + (int64_t)m * K + k0);
      const u32x4 p = *reinterpret_cast<const u32x4*>(iperm + k0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xr[p[q] & 0xFFFFu] = (uint16_t)(v[q] & 0xFFFFu);
        xr[p[q] >> 16] = (uint16_t)(v[q] >> 16);
      }
    } else if (k0 < Kp) {
      *reinterpret_cast<u32x4*>(xr + k0) = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

hipError_t launch_prep(const GemmCall& c, bool to_f16) {
  const gptq_layer* L = c.L;
  uint8_t* base = reinterpret_cast<uint8_t*>(c.ws);
  uint16_t* xs = reinterpret_cast<uint16_t*>(base);
  int32_t* rowexp = to_f16 ? reinterpret_cast<int32_t*>(base + ws_xsorted_bytes(L, c.M)) : nullptr;
  const unsigned rows = (unsigned)(c.M < 65535 ? c.M : 65535);
  if (to_f16 && !L->has_perm && L->Kp <= 2048 * 8) {
    hipLaunchKernelGGL(prep_f16_row_kernel<8>, dim3(rows), dim3(256), 0, c.stream,
                       reinterpret_cast<const uint16_t*>(c.x), xs, rowexp, (int)c.M, L->K, L->Kp);
    return hipGetLastError();
  }
  if (!to_f16 && L->has_perm && L->iperm && c.M <= 32) {
    hipLaunchKernelGGL(prep_scatter_kernel, dim3(rows, (unsigned)((L->Kp + 2047) / 2048)), dim3(256), 0, c.stream,
                       reinterpret_cast<const uint16_t*>(c.x), L->iperm, xs, (int)c.M, L->K, L->Kp);
    return hipGetLastError();
  }
  const int span = to_f16 ? L->Kp : 2048;     // multiple of 2048 or the whole row
  const unsigned stripes = (unsigned)((L->Kp + span - 1) / span);
  hipLaunchKernelGGL(prep_kernel, dim3(rows, stripes), dim3(256), 0, c.stream, reinterpret_cast<const uint16_t*>(c.x),
                     L->has_perm ? L->perm : nullptr, xs, rowexp, (int)c.M, L->K, L->Kp, to_f16 ? 1 : 0, span);
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
  const int32_t* rowexp;   // per-row power of two of the fp16 copy (bf16 activations only)
  uint16_t* y;
  float* part;           // split K: [KS][M][N] fp32 partial sums (KS > 1), else NULL
  int ld;
  int M, K, N, KC, CT, G, scale_kind, MB, NB;
  int KS, kcs;           // K slices and chunks per slice (KS = ceil(KC / kcs))
  uint32_t gmagic;       // segment -> group map (see segment_divisor)
  int gshift;
  const void* bias;      // [N] in the scales' dtype (scale_kind), or NULL
};

// Writes a wave's WM x WN accumulator tiles (rows m0 + 16 i + 4 q + r, column tile ct0 + j, lane
// column col) to y.  bf16 outputs (OB) are first multiplied back by 2^rowexp[m]: the exponents of
// a row block come in one 16-byte load per lane, all issued before the first store.  Rows past M
// are dropped by the y resource (their offsets lie past its end), so the stores need no branches.
template <int OB, int WM, int WN>
__device__ __forceinline__ void store_tiles(const TiledArgs& a, const f32x4 (&acc)[WM][WN], int m0, int ct0, int col,
                                            int q) {
  const rsrc_t ry = make_rsrc(a.y, (uint32_t)((int64_t)a.M * a.N * 2));
  u32x4 ex[WM];
  if constexpr (OB) {
    const rsrc_t re = make_rsrc(a.rowexp, (uint32_t)a.M * 4u);
#pragma unroll
    for (int i = 0; i < WM; ++i) ex[i] = load_b128(re, (uint32_t)(m0 + i * 16 + 4 * q) * 4u, 0u);
  }
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    if (ct0 + j >= a.CT) continue;
    const int n = (ct0 + j) * 16 + col;
    const float bn = bias_at(a.bias, a.scale_kind, n);
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + i * 16 + 4 * q + r;
        const uint32_t off = m < a.M ? (uint32_t)(m * a.N + n) * 2u : kOob;
        if constexpr (OB) store_b16(ry, to_out<1>(ldexpf(acc[i][j][r], (int)ex[i][r]) + bn), off);
        else store_b16(ry, to_out<0>(acc[i][j][r] + bn), off);
      }
  }
}

// Split K: the same tiles as fp32 partial sums of slice ks (bf16 rows already multiplied back by
// 2^rowexp), no bias; launch_part_reduce adds the slices in order.
template <int OB, int WM, int WN>
__device__ __forceinline__ void store_part(const TiledArgs& a, const f32x4 (&acc)[WM][WN], int ks, int m0, int ct0,
                                           int col, int q) {
  const int64_t mn = (int64_t)a.M * a.N;
  const rsrc_t rp = make_rsrc(a.part + ks * mn, (uint32_t)(mn * 4));
  u32x4 ex[WM];
  if constexpr (OB) {
    const rsrc_t re = make_rsrc(a.rowexp, (uint32_t)a.M * 4u);
#pragma unroll
    for (int i = 0; i < WM; ++i) ex[i] = load_b128(re, (uint32_t)(m0 + i * 16 + 4 * q) * 4u, 0u);
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
        const uint32_t off = m < a.M ? (uint32_t)(m * a.N + n) * 4u : kOob;
        const float v = OB ? ldexpf(acc[i][j][r], (int)ex[i][r]) : acc[i][j][r];
        store_b32(rp, __builtin_bit_cast(uint32_t, v), off);
      }
  }
}

// x tile of one chunk in LDS: BM rows x 16 pieces of 16 bytes, no padding, piece c of row r at
// slot r * 16 + (c ^ (r & 15)).  Sixteen lanes reading the same piece of sixteen consecutive
// rows (an A operand) then hit sixteen different 16-byte bank groups.  Lane i of a wave's piece j
// fills slot (wave * A_INST + j) * 64 + i of the tile, so each lane simply fetches the global
// piece that belongs in that slot.
// DEPTH = 1: one chunk in flight (two x buffers filled by buffer_load ... lds, the next chunk's
// loads issued during this chunk's compute, then a full wait); DEPTH = 2: two chunks in flight
// (three x buffers and three register stages, each step waiting only for its own chunk's loads).
// With two chunks in flight the x pieces do not come by LDS DMA: each wave loads them into
// registers with the chunk's other loads and writes them to LDS itself.  A count of outstanding
// loads is a sound wait only for register loads, which complete in issue order: on MI355X, with
// the pieces loaded by DMA and the same counted wait, a 64-row tile in eight waves read 16 stale
// rows of x in about half of its calls, while a full wait before every barrier was always right
// and 13-28 % slower.  The buffers are distinct LDS arrays: the compiler then knows that a read of
// one does not wait on a write to another.
template <int BITS, int OB, int WM, int WN, int SEG, int NW, int DEPTH>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(DEPTH == 2 ? 2 : 1)))
tiled_kernel(const TiledArgs a) {
  constexpr int BM = 16 * WM;
  constexpr int NSEG = 4 / SEG;
  constexpr int PARTS = BITS > 4 ? 2 : 1;      // loads per lane per unit (load_unit)
  constexpr uint32_t UNIT_BYTES = 256u * BITS;
  constexpr int A_BYTES = BM * 256;            // one chunk of x for the tile
  constexpr int A_INST = BM / (4 * NW);        // 1 KB LDS loads per wave per chunk
  static_assert(A_INST * NW * 64 == BM * 16, "x tile must split evenly over the waves");
  static_assert(A_INST <= WM && WM >= 1, "one x piece per row block");
  constexpr int UNITS_AT = WM > 2 ? 2 : WM - 1;   // row block after which a chunk's units go out
  static_assert(DEPTH == 1 || DEPTH == 2, "one or two chunks in flight");
  __shared__ __attribute__((aligned(1024))) uint8_t xs[DEPTH == 1 ? 2 : 1][A_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t xs_b[DEPTH == 2 ? A_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t xs_c[DEPTH == 2 ? A_BYTES : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, q = lane >> 4;

  // XCD-aware remap of the linear workgroup id (see the file comment); with split K the slice is
  // the outermost index, so an XCD's workgroups share one slice of x.
  const int tiles = a.MB * a.NB;
  const int total = tiles * a.KS;
  int lid = blockIdx.x;
  if ((total & 7) == 0) lid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int ks = lid / tiles;
  const int mb = (lid - ks * tiles) / a.NB, nb = (lid - ks * tiles) % a.NB;
  const int kc_lo = ks * a.kcs;
  const int kc_hi = min(a.KC, kc_lo + a.kcs);     // never empty: KS = ceil(KC / kcs)
  const int m0 = mb * BM;
  const int ct0 = nb * (NW * WN) + wave * WN;

  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- resources and fixed per-lane offsets -------------------------------------------------
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)((int64_t)a.M * a.ld * 2));
  // x rows hold whole chunks (ld is a multiple of 128: a padded copy is made otherwise)
  uint32_t voff_a[A_INST];
#pragma unroll
  for (int j = 0; j < A_INST; ++j) {
    const int slot = (wave * A_INST + j) * 64 + lane;
    const int r = slot >> 4, c = (slot & 15) ^ (r & 15);
    voff_a[j] = (m0 + r < a.M) ? (uint32_t)((m0 + r) * a.ld + c * 8) * 2u : kOob;
  }
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
  // A operand reads: row i*16 + col, piece 4t + q  ->  byte (col * 16 + ((4t + q) ^ col)) * 16 + i * 4096
  uint32_t a_off[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) a_off[t] = (uint32_t)(col * 16 + ((4 * t + q) ^ col)) * 16u;

  struct Stage {
    uint32_t w[WN][BITS];
    uint32_t rec[WN][NSEG];
    uint32_t s32[WN][NSEG];
    u32x4 x[DEPTH == 2 ? A_INST : 1];   // the wave's x pieces (two chunks in flight)
  };

  // One 1 KB piece (j) of chunk kc's x tile -> LDS buffer xb by DMA (one chunk in flight).
  auto issue_x = [&](int kc, uint8_t* xb, int j) {
    // (the offset goes through a local: passed straight from the array, the host pass of this
    // compiler drops the kernel's launch stub)
    const uint32_t vo = voff_a[j];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rx, (__attribute__((address_space(3))) void*)(xb + (wave * A_INST + j) * 1024), 16, vo,
        (uint32_t)kc * 256u, 0, 0);
  };
  // One piece (j) of chunk kc's x tile -> registers, and a wave's pieces from there -> LDS buffer
  // xb, the same slots (two chunks in flight).
  auto load_xr = [&](int kc, Stage& st, int j) { st.x[j] = load_b128(rx, voff_a[j], (uint32_t)kc * 256u); };
  auto write_x = [&](const Stage& st, uint8_t* xb) {
#pragma unroll
    for (int j = 0; j < A_INST; ++j)
      *reinterpret_cast<u32x4*>(xb + (wave * A_INST + j) * 1024 + lane * 16) = st.x[j];
  };
  // Chunk kc: packed units and metadata -> registers, then (with_x) its x pieces.
  auto issue = [&](int kc, uint8_t* xb, Stage& st, bool with_x) {
#pragma unroll
    for (int j = 0; j < WN; ++j)
      load_unit<BITS, 0>(rw[j], voff_w, voff_w1, (uint32_t)kc * UNIT_BYTES, st.w[j]);
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const int g = segment_group(SEG == 4 ? kc : kc * 4 + s, a.gmagic, a.gshift, a.G);
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        st.rec[j][s] = load_b32(rm[j], voff_m, (uint32_t)g * 64u);
        st.s32[j][s] = load_b32(rs[j], voff_m, (uint32_t)g * 64u);
      }
    }
    if (with_x) {
#pragma unroll
      for (int j = 0; j < A_INST; ++j) {
        if constexpr (DEPTH == 2) load_xr(kc, st, j);
        else issue_x(kc, xb, j);
      }
    }
  };

  auto compute = [&](const uint8_t* xb, const Stage& st, auto&& hook) {
    u32x4 b[WN][4];
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        b[j][t] = build_b<BITS, 0>(st.w[j], t, zero_term<BITS, 0>(zero_of(st.rec[j][t / SEG])));
    float sc[WN][NSEG];
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int s = 0; s < NSEG; ++s) sc[j][s] = scale_of(st.rec[j][s], st.s32[j][s], a.scale_kind);
    if constexpr (SEG == 1) {
      // four scales per chunk: the plain order keeps the wave within four waves per SIMD
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        hook(i);
        u32x4 af[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) af[t] = *reinterpret_cast<const u32x4*>(xb + a_off[t] + i * 4096);
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
          for (int s = 0; s < NSEG; ++s) {
            f32x4 tmp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = s * SEG; t < (s + 1) * SEG; ++t) tmp = mfma16<0>(af[t], b[j][t], tmp);
            acc[i][j] += sc[j][s] * tmp;
          }
      }
      return;
    }
    // Row block i: its A operands were read during block i-1; block i+1's are read now, and
    // block i-1's segment partials are scaled into acc while block i's MFMAs run.
    u32x4 afc[4], afn[4];
    f32x4 prev[WN][NSEG];
#pragma unroll
    for (int t = 0; t < 4; ++t) afc[t] = *reinterpret_cast<const u32x4*>(xb + a_off[t]);
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      hook(i);
      if (i + 1 < WM) {
#pragma unroll
        for (int t = 0; t < 4; ++t) afn[t] = *reinterpret_cast<const u32x4*>(xb + a_off[t] + (i + 1) * 4096);
      }
      f32x4 part[WN][NSEG];
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int s = 0; s < NSEG; ++s) {
          f32x4 tmp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = s * SEG; t < (s + 1) * SEG; ++t) tmp = mfma16<0>(afc[t], b[j][t], tmp);
          part[j][s] = tmp;
        }
      if (i > 0) {
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
          for (int s = 0; s < NSEG; ++s) acc[i - 1][j] += sc[j][s] * prev[j][s];
      }
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int s = 0; s < NSEG; ++s) prev[j][s] = part[j][s];
#pragma unroll
      for (int t = 0; t < 4; ++t) afc[t] = afn[t];
    }
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int s = 0; s < NSEG; ++s) acc[WM - 1][j] += sc[j][s] * prev[j][s];
  };

  if constexpr (DEPTH == 2) {
    // Chunk c (c = 0, 1, ... from kc_lo) sits in buffer and register stage c % 3.  The step of
    // chunk c waits until at most one chunk's loads (c + 1) are pending, meets the workgroup at the
    // barrier (every wave's x pieces of chunk c are then in LDS, and every wave is done with chunk
    // c - 1), requests chunk c + 2 into stage (c + 2) % 3 while it computes, and at its end writes
    // its pieces of chunk c + 1 (loaded during step c - 1) to buffer (c + 1) % 3, last read in step
    // c - 2.  Requests past the slice repeat its last chunk (L2 hits), so every step of the loop
    // issues the same loads and the wait count is fixed; the last one or two steps after the loop
    // issue nothing and wait for everything.
    constexpr int NL = WN * PARTS + 2 * NSEG * WN + A_INST;   // loads per chunk per wave
    static_assert(NL < 64, "vmcnt holds at most 63");
    Stage st0, st1, st2;
    const int n = kc_hi - kc_lo;
    issue(kc_lo, nullptr, st0, true);
    issue(kc_lo + (n > 1 ? 1 : 0), nullptr, st1, true);
    write_x(st0, &xs[0][0]);                 // (the compiler waits for the pieces' own loads)
    auto step = [&](int c, const Stage& st, const uint8_t* xb, Stage& stn, const Stage& stx, uint8_t* xbx) {
      __builtin_amdgcn_sched_barrier(0);     // no instruction crosses a step boundary
      // this wave's loads of chunk c are in (register loads complete in issue order), and its
      // writes of chunk c's pieces and reads of chunk c - 1 (lgkmcnt); the barrier publishes the
      // pieces with every other wave's.  No fence: a workgroup fence would wait for every load in
      // flight.
      wait_vmcnt<NL>();
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt left alone
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const int kn = kc_lo + min(c + 2, n - 1);
      compute(xb, st, [&](int i) {
        if (i < A_INST) load_xr(kn, stn, i);
        if (i == UNITS_AT) issue(kn, nullptr, stn, false);
      });
      write_x(stx, xbx);
    };
    int c = 0;
    for (; c + 2 < n; c += 3) {
      step(c, st0, &xs[0][0], st2, st1, xs_b);
      step(c + 1, st1, xs_b, st0, st2, xs_c);
      step(c + 2, st2, xs_c, st1, st0, &xs[0][0]);
    }
    if (c < n) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      compute(&xs[0][0], st0, [](int) {});
      if (c + 1 < n) write_x(st1, xs_b);
    }
    if (c + 1 < n) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      compute(xs_b, st1, [](int) {});
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (a.part) store_part<OB, WM, WN>(a, acc, ks, m0, ct0, col, q);
    else store_tiles<OB, WM, WN>(a, acc, m0, ct0, col, q);
    return;
  }

  Stage cur, nxt;
  issue(kc_lo, &xs[0][0], cur, true);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = kc_lo; it < kc_hi; ++it) {
    const int buf = (it - kc_lo) & 1;
    const bool more = it + 1 < kc_hi;
    // The next chunk's x tile goes out one 1 KB piece per row block and its units and metadata
    // after the third piece, so the workgroup's requests do not all queue up at once behind the
    // barrier (measured on MI355X: 5 % faster than issuing everything before the chunk).
    const int kn = more ? it + 1 : it;
    compute(&xs[buf][0], cur, [&](int i) {
      if (i < A_INST) issue_x(kn, &xs[buf ^ 1][0], i);
      if (i == UNITS_AT) issue(kn, &xs[buf ^ 1][0], nxt, false);
    });
    // the next chunk's x tile, units and metadata were issued before this chunk's compute
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    cur = nxt;
  }

  if (a.part) store_part<OB, WM, WN>(a, acc, ks, m0, ct0, col, q);
  else store_tiles<OB, WM, WN>(a, acc, m0, ct0, col, q);
}

template <int BITS, int OB, int WM, int WN, int SEG, int NW, int DEPTH = 1>
static hipError_t run_tiled(const TiledArgs& a0, hipStream_t s) {
  TiledArgs a = a0;
  a.MB = (a.M + 16 * WM - 1) / (16 * WM);
  a.NB = (a.CT + NW * WN - 1) / (NW * WN);
  hipLaunchKernelGGL((tiled_kernel<BITS, OB, WM, WN, SEG, NW, DEPTH>), dim3((unsigned)(a.MB * a.NB * a.KS)),
                     dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

// (tile table and plan: plans.h)
static TiledPlan tiled_plan(const gptq_layer* L, int64_t M) {
  return tiled_plan_of(M, L->Kp, L->N, L->bits, L->KC, L->CT, L->seg_steps);
}

int tiled_slice_chunks(const gptq_layer* L, int64_t M) { return tiled_plan(L, M).kcs; }

size_t ws_tiled_part_bytes(const gptq_layer* L, int64_t M) {
  const TiledPlan p = tiled_plan(L, M);
  return p.KS > 1 ? align256((size_t)p.KS * M * L->N * 4) : 0;
}

template <int BITS, int OB>
static hipError_t run_tiled_m(const TiledArgs& a, int tile, int seg, hipStream_t s) {
  if (seg != 4) return run_tiled<BITS, OB, 8, 1, 1, 8>(a, s);
  switch (tile) {
    case 0: return run_tiled<BITS, OB, 16, 2, 4, 8>(a, s);
    case 2: return run_tiled<BITS, OB, 8, 2, 4, 4>(a, s);
    case 3: return run_tiled<BITS, OB, 4, 2, 4, 4>(a, s);
    case 4: return run_tiled<BITS, OB, 8, 2, 4, 8>(a, s);
    case 5:   // (the four-wave form runs out of registers with 7- and 8-bit stages)
      if constexpr (BITS <= 6) return run_tiled<BITS, OB, 4, 2, 4, 4, 2>(a, s);
      else return run_tiled<BITS, OB, 4, 1, 4, 8, 2>(a, s);
    case 6: return run_tiled<BITS, OB, 2, 1, 4, 8, 2>(a, s);
    case 7: return run_tiled<BITS, OB, 1, 2, 4, 4, 2>(a, s);
    case 8: return run_tiled<BITS, OB, 4, 1, 4, 8, 2>(a, s);
    default: return run_tiled<BITS, OB, 8, 1, 4, 8>(a, s);
  }
}

template <int OB>
static hipError_t run_tiled_bits(const TiledArgs& a, int bits, int tile, int seg, hipStream_t s) {
  switch (bits) {
    case 2: return run_tiled_m<2, OB>(a, tile, seg, s);
    case 3: return run_tiled_m<3, OB>(a, tile, seg, s);
    case 4: return run_tiled_m<4, OB>(a, tile, seg, s);
    case 5: return run_tiled_m<5, OB>(a, tile, seg, s);
    case 6: return run_tiled_m<6, OB>(a, tile, seg, s);
    case 7: return run_tiled_m<7, OB>(a, tile, seg, s);
    default: return run_tiled_m<8, OB>(a, tile, seg, s);
  }
}

// Rows are processed in slices small enough that every byte offset inside a slice (x rows of up
// to 2^20 inputs, y rows of up to 2^20 outputs) fits the 32-bit buffer offsets the kernels use.
hipError_t launch_tiled(const GemmCall& c) {
  const gptq_layer* L = c.L;
  TiledArgs a;
  const uint16_t* x;
  const int32_t* rowexp = nullptr;
  if (tiled_needs_xsorted(L, c.x_bf16)) {
    hipError_t e = launch_prep(c, c.x_bf16 != 0);
    if (e != hipSuccess) return e;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(c.ws);
    x = reinterpret_cast<const uint16_t*>(base);
    if (c.x_bf16) rowexp = reinterpret_cast<const int32_t*>(base + ws_xsorted_bytes(L, c.M));
    a.ld = L->Kp;
  } else {
    x = reinterpret_cast<const uint16_t*>(c.x);
    a.ld = L->K;
  }
  a.wq = L->wq;
  a.meta = L->meta;
  a.scale32 = L->scale32;
  a.K = L->K; a.N = L->N; a.KC = L->KC; a.CT = L->CT; a.G = L->G;
  segment_divisor(L, &a.gmagic, &a.gshift);
  a.scale_kind = L->scales_dtype;
  a.bias = c.bias;
  a.MB = a.NB = 0;
  const TiledPlan p = tiled_plan(L, c.M);
  a.KS = p.KS;
  a.kcs = p.kcs;
  a.part = nullptr;
  if (p.KS > 1) {
    uint8_t* base = reinterpret_cast<uint8_t*>(c.ws);
    if (tiled_needs_xsorted(L, c.x_bf16)) base += ws_xsorted_bytes(L, c.M);
    if (c.x_bf16) base += ws_rowexp_bytes(c.M);
    a.part = reinterpret_cast<float*>(base);
  }
  // rows per slice: x and y byte offsets inside a slice stay below 2^31 (at least 768 rows, as
  // K, N <= 2^20)
  const int64_t lim = ((int64_t(1) << 31) - 1) / (2 * (int64_t)(a.ld > a.N ? a.ld : a.N));
  const int64_t slice = lim / 256 * 256;
  for (int64_t m0 = 0; m0 < c.M; m0 += slice) {
    a.M = (int)(c.M - m0 < slice ? c.M - m0 : slice);
    a.x = x + m0 * a.ld;
    a.rowexp = rowexp ? rowexp + m0 : nullptr;
    a.y = reinterpret_cast<uint16_t*>(c.y) + m0 * a.N;
    hipError_t e = c.x_bf16 ? run_tiled_bits<1>(a, L->bits, p.tile, L->seg_steps, c.stream)
                            : run_tiled_bits<0>(a, L->bits, p.tile, L->seg_steps, c.stream);
    if (e == hipSuccess && a.part)      // (split K implies one row slice)
      e = launch_part_reduce(a.part, a.y, a.M, a.N, a.KS, c.bias, L->scales_dtype, c.x_bf16, c.stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gq
