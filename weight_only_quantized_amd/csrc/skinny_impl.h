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
#pragma once
#include <hip/hip_runtime.h>

#include "bufmem.h"
#include "dequant.h"
#include "internal.h"
#include "plans.h"

namespace gq {

struct SkinnyArgs {
  const uint32_t* wq;
  const uint32_t* meta;   // per (tile, group, column): scale bits | stored zero << 16
  const uint32_t* scale32;  // f32 scale bits (scale_kind == 2 only)
  const uint16_t* x;      // [M, ld] activations (original order when perm is set, else sorted)
  const uint16_t* iperm;  // input index -> sorted position (16-bit), or NULL (identity); LDS staging only
  uint16_t* y;            // [M, N]
  int64_t ld;             // row stride of x in elements
  int M, K, Kp, N, KC, CT, G, scale_kind;
  int Kx;                 // length of a staged x row in LDS: Kp, or the launch's waves per column
                          // group times their chunks times 128 when the last wave's range runs past Kp
  uint32_t gmagic;        // segment -> group map (segment_divisor): min(segment / d, G - 1)
  int gshift;
  const void* bias;       // [N] in the scales' dtype (scale_kind), or NULL
  int cgs;                // column groups per workgroup of the copy form (KSPLIT = 0, XLDS = 3)
};

// Workgroups are handed to the eight XCDs in turn (workgroup i to XCD i mod 8).  This renumbers
// them so that each XCD takes one contiguous run of workgroup numbers, hence of column tiles and of
// the tile-major weight bytes: XCD x, holding the workgroups x, x + 8, x + 16, ..., takes the run
// that starts at x * q + min(x, r) (q, r = nb / 8, nb % 8).  A bijection of [0, nb).  Measured on
// MI355X for a plain 8 KB-per-wave read of 122 MB: 512-thread workgroups 21.7 us in launch order,
// 19.4 us renumbered (256-thread workgroups: 19.2 us in launch order).
__device__ __forceinline__ int xcd_contiguous_block() {
  const int nb = gridDim.x, i = blockIdx.x;
  const int x = i & 7, l = i >> 3, q = nb >> 3, r = nb & 7;
  return x * q + (x < r ? x : r) + l;
}

// Group of segment `si` (a chunk index when segments are chunks, a 32-input step index when they
// are steps).  Every operand is wave-uniform, so this runs on the scalar unit.
template <bool NB = false>
__device__ __forceinline__ int segment_group(int si, uint32_t gmagic, int gshift, int G) {
  return NB ? group_of_segment_nb(si, gmagic, gshift, G) : group_of_segment(si, gmagic, gshift, G);
}

// XLDS = 1: each wave first copies the part of x[0:M, 0:Kp] that its own K range multiplies into
// LDS (rows padded by 16 bytes) and reads its A operands from there, with no workgroup barrier.  XLDS = 0: each chunk's A
// operands are loaded from global memory (L2-resident) one chunk ahead.
// DEPTH chunks of packed weights (and their group metadata) are kept in flight per wave in a
// register ring, so a wave never waits on HBM latency more than once per DEPTH chunks.
// All loads go through buffer resources (bufmem.h): a lane's offset is fixed, the chunk offset is
// a scalar, and the loaded values are only touched at compute time -- an operation on a loaded
// value right after its load (or at a branch join) would force a wait for every load in flight.
// TCH > 0: every wave owns exactly TCH chunks (the dispatcher guarantees KC == KSPLIT * TCH) and
// its whole K range is emitted as straight-line code, so each chunk waits only for its own loads
// (a loop back-edge would make the compiler wait for every load in flight).
// KSPLIT == 0: the number of waves per column tile is the launch's (blockDim.x / 64, at most 16),
// each owning TCH chunks; chunks past the layer's last (the tail of the last wave) are padding:
// their weight loads fall outside the tile's buffer resource and read zeros, their x is staged as
// zeros (the staged row holds Kx inputs), so they add exactly nothing.
// XLDS == 3: the workgroup copies all of x[0:M, 0:Kp] into LDS rows (1 KB buffer_load ... lds pieces,
// Kp a multiple of 512) after issuing its weight ring, and every column group's waves read their A
// operands there: one copy of x per workgroup, shared by its CGS column groups.
// XLDS == 2: an act-order layer; the workgroup scatters all of x into sorted order in LDS through
// the 16-bit inverse permutation, then meets at a barrier (with KSPLIT == 0, M = 1 only: each
// thread then holds TCH / 4 pieces of the padded row).
// At least two waves per SIMD: the kernel needs about 60-130 VGPRs, and without the hint the
// compiler spreads a one-wave-per-SIMD schedule over all 512, so a compute unit held one workgroup.
// ONE (M = 1, whole-chunk segments, x staged per wave, straight-line ranges): the B operand is
// bias + code with no zero subtraction (build_b_offset), and the term -(bias + zero) * sum_k x[k]
// of each chunk is applied to the fp32 partial instead; each wave sums its chunks of x once while
// staging them and keeps the sums in LDS.  Only row 0 of the accumulators is carried.
// F32S: the layer's scales are float32 (a parallel array of scale bits); otherwise the 16-bit scale
// sits in the metadata record and no second load is issued per chunk (2 % on the 8192-input M = 1
// and M = 4 calls on MI355X).
template <int BITS, int XT, int MT, int TW, int KSPLIT, int SEG, int XLDS, int DEPTH, int TCH, int ONE = 0,
          int F32S = 1, int WPE = 2, int NWV0 = 0, int XMAP = 1, int NBS = 0, int PH = 1>
__global__ void __launch_bounds__(64 * (NWV0 ? NWV0 : (KSPLIT == 0 ? 16 : (KSPLIT > 4 ? KSPLIT : 4))))
__attribute__((amdgpu_waves_per_eu(WPE)))
skinny_kernel(const SkinnyArgs a) {
  static_assert(ONE != 1 || (MT == 1 && SEG == 4 && XLDS == 1 && TCH > 0 && (XT == 0 || BITS <= 4)),
                "the M = 1 form needs whole-chunk segments, per-wave staging and an exact offset operand");
  static_assert(PH == 1 || ((PH == 2 || PH == 4) && XLDS == 3 && KSPLIT == 0 && TCH % (4 * PH) == 0),
                "copy phases: the copy form's launch-set waves, at least four chunks per phase");
  static_assert(ONE != 2 || (MT <= 2 && SEG == 4 && XLDS == 3 && TCH > 0 && XT == 1 && BITS <= 4),
                "the offset form for up to 32 rows needs whole-chunk segments, the workgroup's copy of x and "
                "an exact bf16 offset operand");
  constexpr bool RTK = KSPLIT == 0;             // waves per tile set at launch
  static_assert(!RTK || (TCH >= 4 && XLDS != 0), "launch-set K split: per-wave ranges, staged x");
  constexpr int NWV = NWV0 ? NWV0 : (RTK ? 16 : (KSPLIT > 4 ? KSPLIT : 4));  // waves per workgroup (at most)
  static_assert(RTK || NWV % KSPLIT == 0, "whole column groups per workgroup");
  constexpr int NT = 64 * NWV;
  constexpr int CGS = RTK ? 1 : NWV / KSPLIT;   // column groups per workgroup (launch-set form: a.cgs)
  constexpr int NSEG = 4 / SEG;                 // fixup segments per chunk
  constexpr int PARTS = BITS > 4 ? 2 : 1;      // loads per lane per unit (load_unit)
  constexpr uint32_t UNIT_BYTES = 256u * BITS;
  constexpr int NR = ONE == 1 ? 1 : 4;           // accumulator registers carried (ONE = 1: output row 0)
  // Group and scale picked without branches (NB): in the copy form, where the branches around the
  // scale conversion ran the registers out (spills), and where the caller asks for it (NBS) for x
  // read from L2 (a branch join waits for the chunk's x loads in flight; measured on MI355X,
  // 5120 x 13824 M = 4: 14.4 -> 11.5 us; 14336 x 4096 M = 8 measured 12.2 -> 13.0, 4096 x 14336
  // M = 4 9.4 -> 10.0, and the M = 1 forms 1 - 6 % slower, so those keep the branches)
  constexpr bool NB = XLDS == 3 || (XLDS == 0 && NBS);
  auto scale_at = [&](uint32_t rec, uint32_t s32) {
    return NB ? scale_of_nb(rec, s32, a.scale_kind) : scale_of(rec, s32, a.scale_kind);
  };
  // reduction slots; the copy form reuses its copy of x for them (after a barrier), which leaves
  // its whole LDS to the copy
  __shared__ float red_s[XLDS == 3 ? 1 : NWV][MT * TW * NR][64];
  extern __shared__ __attribute__((aligned(16))) uint16_t xlds[];
  float (*const red)[MT * TW * NR][64] =
      XLDS == 3 ? reinterpret_cast<float (*)[MT * TW * NR][64]>(xlds) : red_s;

  // Chunk and tile bookkeeping is wave-uniform (scalar registers).
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // launch-set form: blockDim.x / 64 waves; the copy form (XLDS = 3) splits them into a.cgs column
  // groups of nks waves, the others have one group (no division on the way to the first load)
  constexpr bool GROUPS = RTK && XLDS == 3;
  const int nwaves = RTK ? (int)(blockDim.x >> 6) : NWV;
  const int nks = RTK ? (GROUPS ? nwaves / a.cgs : nwaves) : KSPLIT;   // waves sharing a group's tiles
  const int cg = RTK ? (GROUPS ? wave / nks : 0) : wave / KSPLIT;
  const int ks = RTK ? wave - cg * nks : wave % KSPLIT;
  const int ct0 = ((XMAP ? xcd_contiguous_block() : (int)blockIdx.x) * (GROUPS ? a.cgs : CGS) + cg) * TW;
  const int cpw = RTK ? TCH : (a.KC + KSPLIT - 1) / KSPLIT;
  const int kc0 = ks * cpw;
  const int kc1 = min(a.KC, kc0 + cpw);
  const int col = lane & 15, q = lane >> 4;
  // PH = 2 or 4 (the copy form when x[0:M, 0:Kx] does not fit the LDS): the workgroup copies the
  // first PH-th of the inputs, every wave takes the first T / PH of its chunks from there, and after
  // a barrier the next part replaces it; a wave's chunks are the T / PH of its slot in each part
  const int Kxs = a.Kx / PH;                    // staged inputs per row
  const int xrow = Kxs + 8;                     // LDS row stride (halves)

  f32x4 acc[MT][TW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < TW; ++i) acc[m][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 nb;
  nb[0] = nb[1] = nb[2] = nb[3] = Bias<BITS, XT>::neg2;

  // One resource per tile (units, metadata records, f32 scales); tiles past the end of N alias
  // the last tile -- they are computed but never stored.
  rsrc_t rw[TW], rm[TW], rs[TW];
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const int64_t cti = min(ct0 + i, a.CT - 1);
    rw[i] = make_rsrc(a.wq + cti * a.KC * (64 * BITS), (uint32_t)a.KC * UNIT_BYTES);
    rm[i] = make_rsrc(a.meta + cti * a.G * 16, (uint32_t)a.G * 64u);
    rs[i] = make_rsrc(a.scale32 ? a.scale32 + cti * a.G * 16 : a.meta, a.scale32 ? (uint32_t)a.G * 64u : 0u);
  }
  const uint32_t voff_w = unit_voff0<BITS>(lane), voff_w1 = unit_voff1<BITS>(lane);
  const uint32_t voff_m = (uint32_t)col * 4u;

  struct WChunk {
    uint32_t w[TW][BITS];
    uint32_t rec[TW][NSEG];      // metadata record
    uint32_t s32[TW][NSEG];      // f32 scale bits
  };
  auto load_w = [&](int kc, WChunk& c) {
#pragma unroll
    for (int i = 0; i < TW; ++i)
      load_unit<BITS, kAuxStream>(rw[i], voff_w, voff_w1, (uint32_t)kc * UNIT_BYTES, c.w[i]);
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const int g = segment_group<NB>(SEG == 4 ? kc : kc * 4 + s, a.gmagic, a.gshift, a.G);
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        c.rec[i][s] = load_b32(rm[i], voff_m, (uint32_t)g * 64u);
        if constexpr (F32S) c.s32[i][s] = load_b32(rs[i], voff_m, (uint32_t)g * 64u);
        else c.s32[i][s] = 0u;
      }
    }
  };

  struct XChunk { u32x4 xa[MT][4]; };
  // global A operands: lane (row m*16 + col, k = 128 kc + 32 t + 8 q); rows >= M read 0
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)((int64_t)a.M * a.ld * 2));
  uint32_t voff_x[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int row = m * 16 + col;
    voff_x[m] = row < a.M ? (uint32_t)(row * a.ld + 8 * q) * 2u : kOob;
  }
  auto load_x_global = [&](int kc, XChunk& c) {
    const bool tail = (kc + 1) * kChunkK > a.K;   // last chunk of a K that is not a multiple of 128
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t vo = voff_x[m] + 64u * t;
        if (tail && kc * kChunkK + 32 * t + 8 * q >= a.K) vo = kOob;
        c.xa[m][t] = load_b128(rx, vo, (uint32_t)kc * 256u);
      }
  };
  // A-operand rows >= M read staged row 0: an MFMA output row depends on its own A row only, and
  // output rows >= M are never stored, so they need no zero row (which would double the LDS of an
  // M = 1 call and halve the workgroups a compute unit holds).  Every lane's address is its fixed
  // base plus the chunk offset (an immediate in the straight-line variants).
  int xbase[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xbase[m] = ((m * 16 + col < a.M) ? (m * 16 + col) * xrow : 0) + 8 * q;
  auto load_x_lds = [&](int kc, XChunk& c) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        c.xa[m][t] = *reinterpret_cast<const u32x4*>(&xlds[xbase[m] + kc * kChunkK + 32 * t]);
  };

  // per-chunk sums of x (ONE): TCH floats per wave after the staged rows
  float* const xsum = reinterpret_cast<float*>(xlds + (XLDS ? a.M * xrow : 0)) + wave * TCH;
  // ONE = 2: per-(chunk, row) sums of the workgroup's copy of x, [KC][16] floats after the rows
  float* const xs2 = reinterpret_cast<float*>(xlds + (XLDS ? a.M * xrow : 0));
  auto compute_one = [&](const WChunk& c, const XChunk& xc, int kc) {
    if constexpr (ONE == 2) {
      // rows m * 16 + 4q .. + 3 of this lane's accumulators; rows >= M repeat row 0 and are never
      // stored; each B operand serves every row block
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        u32x4 b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = build_b_offset<BITS, XT>(c.w[i], t);
        const float off = 128.f + (float)zero_of(c.rec[i][0]);
        const float sc = scale_at(c.rec[i][0], c.s32[i][0]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const f32x4 sx = *reinterpret_cast<const f32x4*>(xs2 + (kc * MT + m) * 16 + 4 * q);
          f32x4 tmp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) tmp = mfma16<XT>(xc.xa[m][t], b[t], tmp);
          acc[m][i] += sc * (tmp - off * sx);
        }
      }
    } else if constexpr (ONE) {
      const float sx = xsum[kc - kc0];
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        f32x4 tmp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) tmp = mfma16<XT>(xc.xa[0][t], build_b_offset<BITS, XT>(c.w[i], t), tmp);
        const float off = (XT == 0 ? 1024.f : 128.f) + (float)zero_of(c.rec[i][0]);
        acc[0][i][0] += scale_of(c.rec[i][0], c.s32[i][0], a.scale_kind) * (tmp[0] - off * sx);
      }
    }
  };
  auto compute = [&](const WChunk& c, const XChunk& xc) {
    f32x4 c0[MT][NSEG];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int s = 0; s < NSEG; ++s) {
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (Bias<BITS, XT>::any) {
#pragma unroll
          for (int t = s * SEG; t < (s + 1) * SEG; ++t) v = mfma16<XT>(xc.xa[m][t], nb, v);
        }
        c0[m][s] = v;
      }
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      u32x4 b[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) b[t] = build_b<BITS, XT>(c.w[i], t, zero_term<BITS, XT>(zero_of(c.rec[i][t / SEG])));
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < NSEG; ++s) {
          f32x4 tmp = c0[m][s];
#pragma unroll
          for (int t = s * SEG; t < (s + 1) * SEG; ++t) tmp = mfma16<XT>(xc.xa[m][t], b[t], tmp);
          acc[m][i] += scale_at(c.rec[i][s], c.s32[i][s]) * tmp;
        }
    }
  };

  // ---- prologue ----------------------------------------------------------------------------
  // x staging loads go out before the weight ring (loads complete in issue order).  Act-order
  // layers scatter x into sorted order in LDS through the inverse permutation: both global reads
  // stay coalesced and independent, and the scatter is eight 2-byte LDS writes per piece.
  // (the launch-set form holds one row of Kx = waves * TCH * 128 inputs over 64 * waves threads)
  constexpr int XPT = RTK ? TCH / 4 : 4 * 256 / NT;   // 16-byte x pieces per thread held in registers
  constexpr bool PERMUTE = XLDS == 2;
  const int nthr = RTK ? (int)blockDim.x : NT;
  u32x4 xreg[PERMUTE ? XPT : 1];
  u32x4 ipreg[PERMUTE ? XPT : 1];                 // eight 16-bit sorted positions per piece
  const int per_row = a.Kx / 8;
  const int n8 = XLDS ? a.M * per_row : 0;        // 16-byte pieces of x (original order if iperm)
  // Without act-order each wave stages only the inputs of its own K range (rows 0..M-1), so no wave
  // waits for another before its first chunk.  x_fits_lds bounds a wave's M * wpr row pieces by
  // 64 * XLW (a fixed count of loads: a load under a branch would make the compiler wait for it at
  // once).  With TCH > 0
  // every wave owns exactly TCH chunks, so the piece -> (row, input) split is a shift.
  constexpr int XLW = XLDS == 1 ? (TCH > 0 ? 4 : 8) : 1;
  const int wpr = TCH > 0 ? TCH * (kChunkK / 8) : max(kc1 - kc0, 0) * (kChunkK / 8);
  const int wrows = a.M * wpr;                          // pieces loaded from x
  u32x4 xw[XLW];
  if constexpr (XLDS == 1) {
#pragma unroll
    for (int r = 0; r < XLW; ++r) {
      const int idx = lane + 64 * r;
      const int m = idx / wpr, j0 = kc0 * kChunkK + (idx - m * wpr) * 8;
      const bool real = idx < wrows && j0 < a.K;
      xw[r] = load_b128(rx, real ? (uint32_t)(m * a.ld + j0) * 2u : kOob, 0u);
    }
  }
  if constexpr (XLDS == 2) {
    const rsrc_t rip = make_rsrc(a.iperm, (uint32_t)a.K * 2u);
#pragma unroll
    for (int r = 0; r < XPT; ++r) {
      const int idx = threadIdx.x + nthr * r;
      const int m = idx / per_row, j0 = (idx % per_row) * 8;
      const bool real = idx < n8 && j0 < a.K;
      xreg[r] = load_b128(rx, real ? (uint32_t)(m * a.ld + j0) * 2u : kOob, 0u);
      ipreg[r] = load_b128(rip, real ? (uint32_t)j0 * 2u : kOob, 0u);
    }
  }
  // With TCH > 0 the waves of neighbouring column tiles walk their K ranges from different
  // starting chunks, so at any moment they read different offsets within their units.
  const int rot = (TCH > 0 && PH == 1) ? (ct0 * 5) & (TCH - 1) : 0;
  const int kch = Kxs >> 7;                     // chunks per copy phase
  auto chunk_at = [&](int j) {
    if constexpr (PH > 1) return (j / (TCH / PH)) * kch + ks * (TCH / PH) + (j % (TCH / PH));
    return kc0 + ((j + rot) & (TCH > 0 ? TCH - 1 : 0));
  };
  // the copy form's copy of phase h (inputs h * Kxs .. (h + 1) * Kxs - 1 of every row, zeros past
  // K) and, for the offset form, the sums of each of its chunks' rows, by MFMA against an all-ones
  // operand (the products are exact, the sums fp32 as in the multiply itself)
  auto copy_issue = [&](int h) {
    const int per_row = Kxs >> 9;
    const int n_inst = a.M * per_row;
    for (int d = wave; d < n_inst; d += nwaves) {
      const int r = d / per_row, pc = d - r * per_row;
      const int k = h * Kxs + pc * 512 + lane * 8;
      const uint32_t vo = k < a.K ? (uint32_t)(r * a.ld + k) * 2u : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(xlds + r * xrow + pc * 512), 16, vo, 0u, 0, 0);
    }
  };
  // Everything this wave has in flight is waited for: a count of outstanding loads tells nothing
  // about LDS DMA (buffer_load ... lds), whose completion is not ordered with register loads
  // (MI355X: a tiled kernel whose counted wait relied on that order read stale rows of x).
  auto copy_finish = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    // every wave's share of the copy has landed before any wave reads x (LDS-only fences)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (ONE == 2) {
      u32x4 ones;
      ones[0] = ones[1] = ones[2] = ones[3] = XT == 1 ? 0x3F803F80u : 0x3C003C00u;
      for (int kc = wave; kc < kch; kc += nwaves) {   // padding chunks: sums of zeros
        XChunk xc;
        load_x_lds(kc, xc);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) v = mfma16<XT>(xc.xa[m][t], ones, v);
          if (col == 0) *reinterpret_cast<f32x4*>(xs2 + (kc * MT + m) * 16 + 4 * q) = v;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the copy form's copy goes out first (L2 hits) and the weight ring right behind it, so that the
  // wait for both takes about one HBM latency
  if constexpr (XLDS == 3) {
    copy_issue(0);
    __builtin_amdgcn_sched_barrier(0);
  }
  WChunk ring[DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j)
    if (TCH > 0 || kc0 + j < kc1) load_w(TCH > 0 ? chunk_at(j) : kc0 + j, ring[j]);

  if constexpr (XLDS == 3) copy_finish();

  if constexpr (XLDS == 1) {
#pragma unroll
    for (int r = 0; r < XLW; ++r) {
      if (64 * r < wrows) {                             // wave-uniform
        const int idx = lane + 64 * r;
        if (idx < wrows) {
          const int m = idx / wpr, j0 = kc0 * kChunkK + (idx - m * wpr) * 8;
          *reinterpret_cast<u32x4*>(&xlds[m * xrow + j0]) = xw[r];
        }
      }
    }
    if constexpr (ONE == 1) {
      // piece r of a lane is 8 inputs of chunk kc0 + lane / 16 + 4 r; its 16 lanes add up
#pragma unroll
      for (int r = 0; r < XLW; ++r) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = xw[r][e];
          if constexpr (XT == 0) {
            p += (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
            p += (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
          } else {
            p += __builtin_bit_cast(float, w << 16);
            p += __builtin_bit_cast(float, w & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) p += __shfl_xor(p, o);
        const int ch = lane / 16 + 4 * r;
        if ((lane & 15) == 0 && ch < TCH) xsum[ch] = p;
      }
    }
    // the wave reads back only what it wrote: LDS keeps one wave's accesses in order, the fence
    // keeps the compiler from moving reads above the writes
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  if constexpr (XLDS == 2) {
#pragma unroll
    for (int r = 0; r < XPT; ++r) {
      const int idx = threadIdx.x + nthr * r;
      if (idx < n8) {
        const int m = idx / per_row, j0 = (idx % per_row) * 8;
        if (j0 < a.K) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t sh = 16u * (e & 1);
            const uint16_t h = (uint16_t)(xreg[r][e >> 1] >> sh);
            const int pos = (int)((ipreg[r][e >> 1] >> sh) & 0xFFFFu);
            xlds[m * xrow + pos] = h;
          }
        } else {
          *reinterpret_cast<u32x4*>(&xlds[m * xrow + j0]) = xreg[r];   // zeros past K (and padding)
        }
      }
    }
    // LDS-only fences around the barrier: the weight loads already in flight are not waited for
    // (a workgroup fence on all memory would wait for every load of the ring), and no instruction
    // crosses it (the scheduler would otherwise start the first chunk's dequantisation above it,
    // which waits for that chunk's weights before the wave reaches the barrier)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- main loop: compute chunk kc from the ring slot, then refill the slot with kc + DEPTH ---
  XChunk xcur, xnxt;
  if constexpr (!XLDS) {
    if (kc0 < kc1) load_x_global(TCH > 0 ? chunk_at(0) : kc0, xcur);
  }
  if constexpr (TCH > 0) {
#pragma unroll
    for (int j = 0; j < TCH; ++j) {
      const int kc = chunk_at(j);
      const int kcl = PH > 1 ? kc - (j / (TCH / PH)) * kch : kc;   // chunk within the staged copy
      if constexpr (PH > 1) {
        if (j > 0 && j % (TCH / PH) == 0) {
          // the sums so far are complete here (otherwise the compiler sinks them past the copy
          // below, to their use at the end, and keeps every chunk's partial live until then)
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < TW; ++i) asm volatile("" : "+v"(acc[m][i]));
          // every wave is done with this part before the next replaces it (LDS-only fence: the
          // weights in flight are not waited for here)
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
          copy_issue(j / (TCH / PH));
          copy_finish();
        }
      }
      if constexpr (XLDS == 3) __builtin_amdgcn_sched_barrier(0);   // copy form: LDS reads per chunk
      if constexpr (XLDS) {
        load_x_lds(kcl, xcur);
      } else {
        if (j + 1 < TCH) load_x_global(chunk_at(j + 1), xnxt);
      }
      if constexpr (ONE) compute_one(ring[j % DEPTH], xcur, ONE == 2 ? kcl : kc);
      else compute(ring[j % DEPTH], xcur);
      if (j + DEPTH < TCH) load_w(chunk_at(j + DEPTH), ring[j % DEPTH]);
      if constexpr (!XLDS) xcur = xnxt;
    }
  } else
  for (int base = kc0; base < kc1; base += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      const int kc = base + j;
      if (kc < kc1) {
        if constexpr (XLDS) {
          load_x_lds(kc, xcur);
        } else {
          if (kc + 1 < kc1) load_x_global(kc + 1, xnxt);
        }
        compute(ring[j], xcur);
        if (kc + DEPTH < kc1) load_w(kc + DEPTH, ring[j]);
        if constexpr (!XLDS) xcur = xnxt;
      }
    }
  }

  // ---- reduce the KSPLIT partial sums of each column group, then store ---------------------
  if constexpr (RTK || KSPLIT > 1) {
    if constexpr (XLDS == 3) __syncthreads();   // every wave is done with the copy the slots reuse
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int r = 0; r < NR; ++r) red[wave][(m * TW + i) * NR + r][lane] = acc[m][i][r];
    __syncthreads();
    if (ks != 0) return;
    // unrolled to the workgroup's largest wave count, slots of absent waves masked, so that every
    // LDS read is issued before the first add (a loop bounded at run time waited for each in turn)
#pragma unroll
    for (int w2 = 1; w2 < (RTK ? NWV : KSPLIT); ++w2)   // (launch-set form: slots past nks masked)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const float v = red[GROUPS ? min(wave + w2, NWV - 1) : wave + w2][(m * TW + i) * NR + r][lane];
            acc[m][i][r] += (!RTK || w2 < nks) ? v : 0.f;
          }
  }
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    if (ct0 + i >= a.CT) continue;
    const int n = (ct0 + i) * 16 + col;
    const float bn = bias_at(a.bias, a.scale_kind, n);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m * 16 + 4 * q + r;
        if (row < a.M) a.y[(int64_t)row * a.N + n] = to_out<XT>(acc[m][i][r] + bn);
      }
  }
}

// ------------------------------------------------------------------------------------------------
// Dispatch of one bit width (instantiated in skinny_b<bits>.hip)
// ------------------------------------------------------------------------------------------------
// (the rules that pick a form: plans.h)

template <int BITS, int XT, int MT, int TW, int KSPLIT, int XLDS, int DEPTH, int TCH, int ONE, int F32S,
          int SEG1 = 1,   // SEG1 = 0: whole-chunk groups only (no 32-input-segment kernel is built)
          int WPE = 2,    // minimum waves per SIMD the register allocation must allow
          int NWV0 = 0,   // waves per workgroup (0: max(KSPLIT, 4)); a multiple of KSPLIT
          int XMAP = 1,   // 1: workgroups renumbered XCD-contiguously (xcd_contiguous_block)
          int NBS = 0>    // 1: group and scale picked without branches (x read from L2)
static hipError_t run_tch(const SkinnyArgs& a, int seg, hipStream_t s) {
  constexpr int NWV = NWV0 ? NWV0 : (KSPLIT > 4 ? KSPLIT : 4);
  constexpr int CGS = NWV / KSPLIT;
  const int blocks = (a.CT + TW * CGS - 1) / (TW * CGS);
  // staged rows (+ the per-chunk sums of x of every wave, ONE)
  const size_t lds = (XLDS ? (size_t)a.M * (a.Kx + 8) * 2 : 0) + (ONE ? (size_t)NWV * TCH * 4 : 0);
  if (seg == 4)
    hipLaunchKernelGGL((skinny_kernel<BITS, XT, MT, TW, KSPLIT, 4, XLDS, DEPTH, TCH, ONE, F32S, WPE, NWV0, XMAP, NBS>), dim3(blocks),
                       dim3(64 * NWV), lds, s, a);
  else if constexpr (TCH == 0 && SEG1)
    hipLaunchKernelGGL((skinny_kernel<BITS, XT, MT, TW, KSPLIT, 1, XLDS, DEPTH, 0, 0, F32S>), dim3(blocks),
                       dim3(64 * NWV), lds, s, a);
  return hipGetLastError();
}

// The M = 1 rule (skinny_m1_rule): one tile per workgroup, ceil(KC / TCH) waves set at launch, all
// of a wave's loads in flight (8-bit codes: four chunks, for the registers), bf16 x in the offset
// form (build_b_offset) for 2/3/4-bit codes.
// The kernel is built for at most 8 or at most 16 waves (the smaller build has half the reduction
// slots: measured on MI355X, the 16-wave build took 4 % longer on the 8-wave 4096 x 14336 call).
template <int BITS, int XT, int TCH, int F32S>
static hipError_t run_m1(const SkinnyArgs& a0, hipStream_t s) {
  constexpr int ONE = XT == 1 && BITS <= 4;
  constexpr int DEPTH = TCH == 16 || (BITS > 4 && TCH > 4) ? 4 : TCH;
  SkinnyArgs a = a0;
  const int waves = (a.KC + TCH - 1) / TCH;
  a.Kx = waves * TCH * kChunkK;
  const size_t lds = (size_t)(a.Kx + 8) * 2 + (ONE ? (size_t)16 * TCH * 4 : 0);
  if (waves <= 8)
    hipLaunchKernelGGL((skinny_kernel<BITS, XT, 1, 1, 0, 4, 1, DEPTH, TCH, ONE, F32S, 2, 8>), dim3(a.CT),
                       dim3(64 * waves), lds, s, a);
  else
    hipLaunchKernelGGL((skinny_kernel<BITS, XT, 1, 1, 0, 4, 1, DEPTH, TCH, ONE, F32S, 2, 16>), dim3(a.CT),
                       dim3(64 * waves), lds, s, a);
  return hipGetLastError();
}

template <int BITS, int XT, int TCH, int F32S>
static hipError_t run_m1_act(const SkinnyArgs& a0, hipStream_t s) {
  SkinnyArgs a = a0;
  const int waves = (a.KC + TCH - 1) / TCH;   // at most 8 (KC <= 64, T = 8 or 16; KC <= 32, T = 4)
  a.Kx = waves * TCH * kChunkK;
  const size_t lds = (size_t)(a.Kx + 8) * 2;
  hipLaunchKernelGGL((skinny_kernel<BITS, XT, 1, 1, 0, 4, 2, 4, TCH, 0, F32S, 2, 8>), dim3(a.CT), dim3(64 * waves),
                     lds, s, a);
  return hipGetLastError();
}

template <int BITS, int XT, int TCH, int F32S, int PH, int MT>
static hipError_t run_copy(const SkinnyArgs& a0, const CopyPlan& p, hipStream_t s) {
  constexpr int ONE = XT == 1 ? 2 : 0;
  SkinnyArgs a = a0;
  a.Kx = p.nks * TCH * kChunkK;
  a.cgs = p.cgs;
  const int blocks = (a.CT + p.cgs - 1) / p.cgs;
  hipLaunchKernelGGL((skinny_kernel<BITS, XT, MT, 1, 0, 4, 3, 4, TCH, ONE, F32S, 2, (MT == 1 ? 16 : 8), 1, 0, PH>), dim3(blocks),
                     dim3(64 * p.cgs * p.nks), p.lds, s, a);
  return hipGetLastError();
}

template <int BITS, int XT, int MT, int TW, int KSPLIT, int XLDS, int DEPTH, int F32S>
static hipError_t run(const SkinnyArgs& a, int seg, hipStream_t s) {
  // Straight-line variants for the whole-chunk-segment case; ring depths measured best on
  // MI355X for 4-bit M=1 (2 for 8 chunks per wave, 4 for 16).
  if (seg == 4 && a.KC == 4 * KSPLIT)
    return run_tch<BITS, XT, MT, TW, KSPLIT, XLDS, (DEPTH < 2 ? DEPTH : 2), 4, 0, F32S>(a, seg, s);
  if (seg == 4 && a.KC == 8 * KSPLIT)
    return run_tch<BITS, XT, MT, TW, KSPLIT, XLDS, (DEPTH < 2 ? DEPTH : 2), 8, 0, F32S>(a, seg, s);
  if (seg == 4 && a.KC == 16 * KSPLIT) return run_tch<BITS, XT, MT, TW, KSPLIT, XLDS, DEPTH, 16, 0, F32S>(a, seg, s);
  return run_tch<BITS, XT, MT, TW, KSPLIT, XLDS, DEPTH, 0, 0, F32S>(a, seg, s);
}

// x staged in LDS whole, or (M <= 16, see skinny_reads_x_from_l2) read from L2 per chunk, two
// column tiles per wave so that x traffic stays near the weight traffic.
template <int BITS, int XT, int F32S>
static hipError_t run_m(const SkinnyArgs& a, int seg, hipStream_t s) {
  if (skinny_m1_rule(a.M, a.KC, seg, a.iperm != nullptr)) {
    const int t = skinny_m1_chunks(a.KC);
    if (t == 4) return run_m1<BITS, XT, 4, F32S>(a, s);
    // (5/6/7-bit codes keep to 8 chunks a wave: 16 with their spare-bit codes exceed the 128
    // VGPRs of a 16-wave workgroup)
    if (t == 8 || (BITS > 4 && BITS < 8)) return run_m1<BITS, XT, 8, F32S>(a, s);
    if constexpr (BITS <= 4 || BITS == 8) return run_m1<BITS, XT, 16, F32S>(a, s);
    return hipErrorInvalidValue;   // (not reached)
  }
  if (skinny_m1_act_rule(a.M, a.Kp, seg, a.iperm != nullptr)) {
    if (a.KC <= 32) return run_m1_act<BITS, XT, 4, F32S>(a, s);
    if constexpr (BITS == 4) return run_m1_act<BITS, XT, 16, F32S>(a, s);
    else return run_m1_act<BITS, XT, 8, F32S>(a, s);
  }
  if (x_fits_lds(a.M, a.Kp)) {
    if (a.iperm) return run<BITS, XT, 1, 1, 4, 2, 4, F32S>(a, seg, s);
    return run<BITS, XT, 1, 1, 4, 1, 4, F32S>(a, seg, s);
  }
  if constexpr (BITS <= 4) {
    const CopyPlan cp = skinny_copy_plan(a.M, a.KC, a.CT, BITS, seg, a.iperm != nullptr);
    if (cp.ok) {
      if (cp.mt == 1) {
        if (cp.ph == 1)
          return cp.T == 16 ? run_copy<BITS, XT, 16, F32S, 1, 1>(a, cp, s) : run_copy<BITS, XT, 32, F32S, 1, 1>(a, cp, s);
        return cp.T == 16 ? run_copy<BITS, XT, 16, F32S, 2, 1>(a, cp, s) : run_copy<BITS, XT, 32, F32S, 2, 1>(a, cp, s);
      }
      if (cp.ph == 1)
        return cp.T == 16 ? run_copy<BITS, XT, 16, F32S, 1, 2>(a, cp, s) : run_copy<BITS, XT, 32, F32S, 1, 2>(a, cp, s);
      if (cp.ph == 2)
        return cp.T == 16 ? run_copy<BITS, XT, 16, F32S, 2, 2>(a, cp, s) : run_copy<BITS, XT, 32, F32S, 2, 2>(a, cp, s);
      return cp.T == 16 ? run_copy<BITS, XT, 16, F32S, 4, 2>(a, cp, s) : run_copy<BITS, XT, 32, F32S, 4, 2>(a, cp, s);
    }
  }
  if (skinny_mx_long(a.M, a.KC, a.CT, seg, a.iperm != nullptr)) {
    if (a.KC < 64) {     // 40 / 48 / 56 chunks: five to seven waves of 8
      if (a.CT >= 512) {
        if (a.KC == 40) return run_tch<BITS, XT, 1, 2, 5, 0, 2, 8, 0, F32S, 0, 2, 0, 1, 1>(a, seg, s);
        if (a.KC == 48) return run_tch<BITS, XT, 1, 2, 6, 0, 2, 8, 0, F32S, 0, 2, 0, 1, 1>(a, seg, s);
        return run_tch<BITS, XT, 1, 2, 7, 0, 2, 8, 0, F32S, 0, 2, 0, 1, 1>(a, seg, s);
      }
      if (a.KC == 40) return run_tch<BITS, XT, 1, 1, 5, 0, 2, 8, 0, F32S, 0, 2, 0, 1, 1>(a, seg, s);
      if (a.KC == 48) return run_tch<BITS, XT, 1, 1, 6, 0, 2, 8, 0, F32S, 0, 2, 0, 1, 1>(a, seg, s);
      return run_tch<BITS, XT, 1, 1, 7, 0, 2, 8, 0, F32S, 0, 2, 0, 1, 1>(a, seg, s);
    }
    if (a.CT >= 512) {
      if (a.KC == 80) return run_tch<BITS, XT, 1, 2, 5, 0, 4, 16, 0, F32S, 0>(a, seg, s);
      if (a.KC == 96) return run_tch<BITS, XT, 1, 2, 6, 0, 4, 16, 0, F32S, 0>(a, seg, s);
      return run_tch<BITS, XT, 1, 2, 7, 0, 4, 16, 0, F32S, 0>(a, seg, s);
    }
    if (a.KC == 80) return run_tch<BITS, XT, 1, 1, 5, 0, 4, 16, 0, F32S, 0>(a, seg, s);
    if (a.KC == 96) return run_tch<BITS, XT, 1, 1, 6, 0, 4, 16, 0, F32S, 0>(a, seg, s);
    return run_tch<BITS, XT, 1, 1, 7, 0, 4, 16, 0, F32S, 0>(a, seg, s);
  }
  if (a.M <= 16) return run<BITS, XT, 1, 2, 4, 0, 4, F32S>(a, seg, s);
  if constexpr (BITS != 2) {
    // two row blocks; M * KC <= 640 leaves at most 37 chunks, so the 16-chunk form is not built
    if (a.M <= 32 && seg == 4) {
      if (a.KC == 16) return run_tch<BITS, XT, 2, 2, 4, 0, 2, 4, 0, F32S>(a, seg, s);
      if (a.KC == 32) return run_tch<BITS, XT, 2, 2, 4, 0, 2, 8, 0, F32S>(a, seg, s);
      return run_tch<BITS, XT, 2, 2, 4, 0, 4, 0, 0, F32S, 0>(a, seg, s);
    }
  }
  return hipErrorInvalidValue;   // larger M goes to the mid family
}

template <int BITS>
hipError_t skinny_bits(const SkinnyArgs& a, int x_bf16, int seg, hipStream_t s) {
  if (a.scale_kind == 2) return x_bf16 ? run_m<BITS, 1, 1>(a, seg, s) : run_m<BITS, 0, 1>(a, seg, s);
  return x_bf16 ? run_m<BITS, 1, 0>(a, seg, s) : run_m<BITS, 0, 0>(a, seg, s);
}
hipError_t skinny_b2(const SkinnyArgs& a, int x_bf16, int seg, hipStream_t s);
hipError_t skinny_b3(const SkinnyArgs& a, int x_bf16, int seg, hipStream_t s);
hipError_t skinny_b4(const SkinnyArgs& a, int x_bf16, int seg, hipStream_t s);
hipError_t skinny_b5(const SkinnyArgs& a, int x_bf16, int seg, hipStream_t s);
hipError_t skinny_b6(const SkinnyArgs& a, int x_bf16, int seg, hipStream_t s);
hipError_t skinny_b7(const SkinnyArgs& a, int x_bf16, int seg, hipStream_t s);
hipError_t skinny_b8(const SkinnyArgs& a, int x_bf16, int seg, hipStream_t s);

}  // namespace gq
