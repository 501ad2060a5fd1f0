// Launch plans of the three kernel families, as functions of the layer's shape and the row count:
// the skinny family's forms (skinny_impl.h launches what they pick), the mid kernel's K slices
// (mid_impl.h) and the tiled family's tile and K split (tiled.hip).  Plain host C++, so that a host
// build can check them (tests/plan_check.cpp).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

#include "layout.h"

namespace gq {

constexpr int kXLdsMax = 64 * 1024;   // dynamic LDS budget for staged x

// True when x for this call can be staged in LDS (small M): the call then needs no workspace.
// The staging holds at most 4 pieces of 8 inputs per thread (M * Kp <= 8192).
inline bool x_fits_lds(int64_t M, int Kp) {
  // (with M * Kp <= 8192, a wave's share (M + 1) * 16 * ceil(Kp / 512) is at most 512 pieces)
  return M <= 4 && M * (int64_t)Kp <= 4 * 8 * 256 && (M + 1) * (int64_t)(Kp + 8) * 2 <= kXLdsMax &&
         (M + 1) * 16 * ((Kp / 128 + 3) / 4) <= 512;
}

// M = 1 without act-order, whole-chunk groups, up to 128 chunks (16384 inputs): one column tile per
// workgroup, whose ceil(KC / T) waves each stage their own T chunks of x in LDS and stream those
// chunks' weights (T = 4 or 8: every load in flight at once; T = 16: four chunks in flight); the
// last wave's chunks past the layer are padding (zeros).  A rule, not a table: any K in range takes
// it.  T = 4 up to 32 chunks, 8 up to 72 chunks or when the chunk count is not a multiple of 16,
// else 16.  Measured on MI355X (us, interleaved on one device): 4096 x 14336 7.69 -> 7.44 against two
// waves of 16 chunks; 8192 x 28672 bf16 22.2 -> 20.46 against four waves of 16; T = 8 vs 16:
// 9216 x 8192 9.38 / 9.71, 11008 x 4096 6.82 / 7.43, 12288 x 8192 10.68 / 11.07 (the one layer the
// rule gives away), 10240 x 8192 9.90 / 9.32, 14336 x 4096 7.94 / 7.73, 16384 x 8192 15.0 / 13.9;
// layers between the exact sizes the previous dispatch knew no longer fall to the split-K mid
// kernel (9216 x 8192: 14.1 -> 9.4; 11008 x 4096: 10.7 -> 6.9).
constexpr int kM1MaxChunks = 128;
inline bool skinny_m1_rule(int64_t M, int KC, int seg_steps, bool has_perm) {
  return M == 1 && !has_perm && seg_steps == 4 && KC <= kM1MaxChunks;
}
inline int skinny_m1_chunks(int KC) { return KC <= 32 ? 4 : (KC <= 72 || KC % 16 != 0 ? 8 : 16); }
// M = 1 with act-order, whole-chunk groups and x staged whole (Kp <= 8192): the same launch-set
// waves, the workgroup scattering x into sorted order through the 16-bit inverse permutation (whose
// within-group order the repack chose so that each scatter instruction hits distinct LDS banks)
// and meeting at one barrier; four chunks in flight per wave.  T = 4 up to 32 chunks, else 16 for
// 4-bit codes and 8 otherwise.  Measured on MI355X, 8192 x 8192, fp16 x, us (the identity-order
// gs = -1 layer of the same width in parentheses): 2-bit 8.6 -> 7.49 (7.10), 3-bit 9.2 -> 8.13
// (7.57), 4-bit 8.9 -> 8.34 (8.01), 8-bit 13.2 -> 12.7 (12.2); before, four waves of 16 chunks
// scattered through a 32-bit inverse permutation in the stable order (about 13 bank-conflict cycles
// per 2-byte LDS write instruction, rocprofv3 SQ_LDS_BANK_CONFLICT) and met at a barrier that also
// waited for every weight load in flight.
inline bool skinny_m1_act_rule(int64_t M, int Kp, int seg_steps, bool has_iperm) {
  return M == 1 && has_iperm && seg_steps == 4 && Kp <= kIpermMaxKp;
}
// 2 <= M <= 32, the copy form (XLDS = 3 with launch-set waves): each workgroup copies x[0:M, 0:Kx]
// into LDS (1 KB buffer_load ... lds pieces), in PH = 2 or 4 parts of the inputs when the whole rows
// do not fit (each part replaces the previous one after a barrier); cgs column groups of one tile
// each share it, and a group's nks waves split K in ranges of T chunks (padding chunks past the
// layer read zeros).  17 to 32 rows are two 16-row blocks sharing every B operand (at most 8 waves:
// the 16-wave bound leaves 128 VGPRs, which two blocks exceed).  bf16 x takes the offset form (128 +
// code, the -(128 + zero) * sum_k x correction from per-chunk, per-row sums the workgroup takes
// once per part by MFMA against an all-ones operand).  Workgroups are sized so that about one round
// of them fills the chip: one per compute unit when the copy takes more than half of the LDS (up to
// 16 waves, 8 with two row blocks), two otherwise (up to 8), and one when two would leave fewer than
// four waves a workgroup; cgs = ceil(CT / (256 x workgroups per compute unit)), T = 16 while that
// many waves fit, else 32; fewer padding chunks than real ones.  Measured on MI355X against the
// previous dispatch (the mid kernel's split K with its reduction launch, or x read from L2), us:
// 8192 x 28672 bf16 M = 2 / 4 / 6 / 8: 26.4 / 27.9 / 28.8 / 30.1 -> 24.2 / 24.9 / 25.5 / 26.2;
// 4096 x 14336 fp16 M = 8 / 12 / 16: 10.2 / 11.3 / 12.7 -> 9.5 / 9.9 / 10.4, M = 17 / 32 (against
// the tiled family) 15.0 / 16.7 -> 11.7 / 13.9; 14336 x 4096 fp16 M = 2 / 4: 11.3 / 11.8 -> 8.7 /
// 9.7; 8192 x 8192 fp16 M = 4: 11.9 -> 9.4.  Act-order layers take it once their x is sorted into
// the workspace (x_unsorted then false).  Not taken: 8-bit codes, 32-input groups, 40 / 48 / 56
// chunks at M <= 8 and up to 32 chunks at M <= 4 (x read from L2 measured faster: 5120 x 13824
// M = 4 / 5 11.5 against 12.2 / 12.3, 4096 x 14336 M = 4 9.4 against 9.8), and shapes for which
// no part count fits the LDS with enough waves (the 8192-input layer at 20 to 32 rows over 1792
// column tiles).
struct CopyPlan {
  bool ok;
  int T, nks, cgs, ph, mt;   // ph: copy phases (parts of the inputs); mt: 16-row blocks
  size_t lds;                // dynamic LDS: the rows and the per-(chunk, row) sums of the offset
                             // form, or the reduction slots that reuse them, whichever is larger
};
inline CopyPlan skinny_copy_plan(int64_t M, int KC, int CT, int bits, int seg_steps, bool x_unsorted) {
  CopyPlan p{false, 0, 0, 0, 1, 1, 0};
  if (M < 2 || M > 32 || bits > 4 || seg_steps != 4 || x_unsorted) return p;
  if ((KC == 40 || KC == 48 || KC == 56) && M <= 8) return p;
  if (KC <= 32 && M <= 4) return p;
  // 17..32 rows over 64 or more chunks go to the tiled family's 32-row tile instead (MI355X, us,
  // copy form -> 32 x 128 tile, whole calls: 8192 x 28672 bf16 M = 17 / 19 38.9 / 39.2 -> 35.2 /
  // 35.7; 8192 x 8192 bf16 4-bit M = 32 20.8 -> 18.1, fp16 M = 20 15.6 -> 14.2, act-order M = 32
  // 2 / 4-bit 20.9 / 21.9 -> 19.3 / 18.5), except 2-bit codes below 20 rows (act-order M = 17
  // 16.5 against 17.7); over 32 chunks the copy form stays ahead (4096 x 14336 M = 24 / 32: 12.6 /
  // 13.5 against 13.8 / 14.4)
  if (M > 16 && KC >= 64 && (bits > 2 || M >= 20)) return p;
  constexpr size_t kLds = 160 * 1024;
  const int mt = M <= 16 ? 1 : 2;
  for (int ph : {1, 2, 4}) {
    if (mt == 1 && ph == 4) break;
    for (int T : {16, 32}) {
      if (T < 4 * ph) continue;
      const int nks = (KC + T - 1) / T;
      const size_t Kxs = (size_t)nks * T * kChunkK / ph;      // inputs per staged row
      size_t lds = (size_t)M * (Kxs + 8) * 2 + (Kxs / kChunkK) * 16 * mt * 4;
      const size_t red = (size_t)16 * mt * 4 * 64 * 4;         // 16 waves' slots, the worst case
      if (lds < red) lds = red;
      if (lds > kLds) continue;
      // two workgroups per compute unit when two copies fit, else (or when that leaves fewer than
      // four waves a workgroup) one
      for (int wpc = lds * 2 <= kLds ? 2 : 1; wpc >= 1; --wpc) {
        // (two row blocks: at most 8 waves, which leaves each of them 256 VGPRs)
        const int W = mt == 2 ? 8 : (wpc == 1 ? 16 : 8);
        int cgs = (CT + 256 * wpc - 1) / (256 * wpc);
        cgs = cgs < 1 ? 1 : (cgs > W ? W : cgs);
        const int nks_max = W / cgs > 0 ? W / cgs : 1;
        // at least four waves a workgroup, and fewer padding chunks than real ones (2048 x 14336
        // at M = 17: two waves of one 16-chunk range measured 12.3 us, four of 32 chunks half
        // padding 13.5, against 9.6 for x read from L2)
        if (nks <= nks_max && nks * cgs >= 4 && nks * T < 2 * KC) return CopyPlan{true, T, nks, cgs, ph, mt, lds};
      }
    }
  }
  return p;
}
// 2 <= M <= 16 on the same layers: the same waves of 16 chunks with x read from L2 per chunk, one
// column tile per wave below 512 column tiles and two from 512 (enough workgroups either way).
// Measured on MI355X against the mid kernel / the tiled family (us): 14336 x 4096, M = 2 / 4 / 8 /
// 12: 9.7 / 10.3 / 12.0 / 14.5 against 14.4 / 14.4 / 14.8 / 15.3; 12288 x 8192, M = 2 / 8 / 16:
// 13.4 / 14.6 / 18.2 against 16.0 / 19.3 / 20.5.  (At 13 to 16 rows on fewer than 512 column tiles
// the tiled family measured faster.)
// 5120 / 6144 / 7168 inputs (40 / 48 / 56 chunks): five to seven waves of 8 chunks, up to M = 8
// (5120 x 5120 M = 2 / 4 / 8: 8.8 / 9.6 / 9.8 -> 7.5 / 8.0 / 9.4 us; 7168 x 20480 M = 8: 24.5 ->
// 23.1 us; slower than the mid kernel from 12 rows).
inline bool skinny_mx_long(int64_t M, int KC, int CT, int seg_steps, bool has_perm) {
  if (M < 2 || has_perm || seg_steps != 4) return false;
  if (KC == 40 || KC == 48 || KC == 56) return M <= 8;
  return M <= (CT >= 512 ? 16 : 12) && (KC == 80 || KC == 96 || KC == 112);
}

// The other case the skinny kernel keeps: x read from L2 per chunk, for M <= 16 over at most 32
// chunks of K, for M <= 4 at any K when the layer has at least 1024 column tiles (enough workgroups
// for its long per-wave ranges), and for 17 <= M <= 32 (two 16-row blocks) while M * KC <= 640.
// Measured on MI355X: faster there than the mid family's split K (8192 x 28672, M = 2 / 3 / 4:
// 28.3 / 29.5 / 30.7 us against 30.1 / 30.5 / 31.2) and than the tiled family (2048 x 14336,
// M = 17 / 32: 9.5 / 12.6 us against 15.0 / 17.3; 4096 x 14336, M = 17 / 20: 15.6 / 16.9 against
// 17.4 / 17.1); slower beyond (14336 x 4096, 256 column tiles, M = 1: 29.3 us against the mid
// kernel's 13.4).
// (The two-block form is built for whole-chunk groups and 3/4/8-bit codes: with 2-bit codes or
// 32-input groups it does not fit its registers.)
inline bool skinny_reads_x_from_l2(int64_t M, int KC, int CT, int bits, int seg_steps) {
  return (M <= 16 && (KC <= 32 || (M <= 4 && CT >= 1024))) ||
         (M > 16 && M <= 32 && M * KC <= 640 && bits != 2 && seg_steps == 4);
}


// ---- mid family ------------------------------------------------------------------------------
// Shape of one mid call: row blocks, K slices and chunks per slice.
struct MidPlan {
  int MT;       // 16-row blocks held (1, 2 or 4)
  int KS;       // K slices (workgroups along K)
  int cpw;      // chunks per slice: 4, 8 or 16
};
constexpr int kMidNW = 4, kMidWN = 2;          // four waves of two column tiles: 128 columns

// Slices of 16, 8 or 4 chunks (x of one slice: cpw * MT * 4 KB <= 64 KB of LDS), the longest that
// still gives two workgroups per compute unit (longer slices stream behind a 2-chunk ring; at four
// workgroups per compute unit the 4-chunk slices loaded everything before computing, 13-16 %
// slower on the act-order 8192 x 8192, M = 32 layer).
// Rows per pass: all of M, except 32 for 32-input segments (whose four-row-block variant would
// not fit in registers).
inline int64_t mid_rows_per_pass_of(int seg_steps) { return seg_steps == 4 ? 64 : 32; }

inline MidPlan mid_plan_of(int64_t M, int KC, int CT, int seg_steps) {
  MidPlan p;
  if (M > mid_rows_per_pass_of(seg_steps)) M = mid_rows_per_pass_of(seg_steps);
  p.MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  const int nbk = (CT + kMidNW * kMidWN - 1) / (kMidNW * kMidWN);
  // one row block starts from 8-chunk slices while that keeps K in at most 8 slices, else from 16
  // (MI355X, bf16 x, M = 8 / 16: the 8192 x 28672 layer 33.4 / 35.1 us with 16-chunk slices,
  // 30.8 / 32.6 with 8; the 28672 x 8192 layer 30.8 / 33.2 with 16, 32.5 / 33.8 with 8, whose 28
  // slices the reduction then adds)
  int cpw = seg_steps == 4 ? (p.MT == 1 ? (KC > 64 ? 16 : 8) : 8 / (p.MT / 2)) : 4;
  while (cpw > 4 && (int64_t)nbk * ((KC + cpw - 1) / cpw) < 2 * 256) cpw /= 2;
  p.cpw = cpw;
  p.KS = (KC + cpw - 1) / cpw;
  return p;
}


// ---- tiled family ----------------------------------------------------------------------------
// Tile table: (rows, columns) of a workgroup tile, its wave tile and wave count.
struct TileShape { int WM, WN, NW; };
constexpr TileShape kTiles[] = {
  {16, 2, 8},   // 0: 256 x 256, wave 256 x 32
  {8, 1, 8},    // 1: 128 x 128, wave 128 x 16 (also every 32-input-segment layer)
  {8, 2, 4},    // 2: 128 x 128, wave 128 x 32
  {4, 2, 4},    // 3:  64 x 128, wave  64 x 32
  {8, 2, 8},    // 4: 128 x 256, wave 128 x 32
  {4, 2, 4},    // 5:  64 x 128 as 3, two chunks in flight (7- and 8-bit codes: as 8)
  {2, 1, 8},    // 6:  32 x 128, wave  32 x 16, two chunks in flight
  {1, 2, 4},    // 7:  16 x 128, wave  16 x 32, two chunks in flight
  {4, 1, 8},    // 8:  64 x 128, wave  64 x 16, two chunks in flight (grids of at most 256)
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

struct TiledPlan { int tile, KS, kcs; };

inline int64_t tiles_of(int64_t M, int CT, int t) {
  const TileShape& ts = kTiles[t];
  return ((M + 16 * ts.WM - 1) / (16 * ts.WM)) * ((CT + ts.NW * ts.WN - 1) / (ts.NW * ts.WN));
}

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Tile and K split of a call: an M-bucketed tile table as in "Formats and kernels ...", section
// "Tile tables, and what happens when your shape does not fit", re-derived for gfx950 from a sweep
// of every tile and split on MI355X (4-bit g128, 4096 x 14336 and 8192 x 28672 layers, M = 4 ..
// 1024): a call runs best with about one eight-wave workgroup (or two four-wave ones) per compute
// unit, from the largest tile that gets there, and splits K only as far as needed to get there:
//   * M <= 16: the 16 x 128 tile, K split the same way (14336 x 4096 M = 16: 13.1 -> 11.8 us,
//     8192 x 28672 fp16 M = 8 / 16 about 10 % faster than the 32 x 128 tile);
//   * M <= 32: the 32 x 128 tile, K split up to ~256 workgroups (MI355X, fp16 x, us, against the
//     64 x 128 tile at its split: 8192 x 28672 M = 24 / 32 37.3 / 38.5 -> 30.5 / 32.2; 8192 x 8192
//     4-bit M = 32 27.5 -> 14.8; 14336 x 4096 M = 16 / 32 -> 13.1 / 14.2 against the dispatch's
//     15.3 / 16.7), in eight waves of 32 x 16 rather than four of 32 x 32 (within 2 % either way
//     on those calls, in about half the registers);
//   * M <= 64: the 64 x 128 tile, K split up to ~448 workgroups;
//   * M <= 512 on layers of at most 4096 inputs whose 64-row blocks together read at most 128 MB
//     of packed weights (the repeated passes then come from the Infinity Cache): the 64 x 128
//     tile too, K split in two below ~192 tiles (4096 x 6144, M = 128 / 512: 24.3 / 52.7 us with
//     the tiles below against 19.1 / 36.7; 4096 x 14336, M = 256: 43.3 against 39.5; longer K or
//     more weight passes measured slower: 14336 x 4096 M = 128 31.2 against 45.3, 8192 x 28672
//     M = 256 120.4 against 148.7);
//   * the 64 x 128 tile in eight waves of 64 x 16 when its grid has at most 256 workgroups
//     (one per compute unit, so four waves would leave every SIMD one wave): 4096 x 14336 M = 128
//     30.5 -> 27.5 us, 4096 x 6144 M = 256 29.4 -> 25.5; on larger grids four waves stay
//     (4096 x 6144 M = 512: 43.3 against 47.9; 8192 x 28672 M = 48 / 64: 51.8 / 54.4 against
//     57.3 / 60.2, where eight waves read every x tile from LDS twice as often);
//   * larger M: the 256 x 256 tile once it alone gives ~192 workgroups, else the 128 x 256 tile,
//     K split up to ~224 workgroups when it gives fewer than ~150;
//   * 32-input segments: the 128 x 128 tile (wave 128 x 16), split the same way.
// Split K only while one slice of partial sums stays addressable by 32-bit offsets and the rows
// are one launch (14336 x 4096 at M = 1024, the 128 x 256 tile unsplit: 179 us; an earlier fixed
// 768-row limit had kept such calls unsplit).
inline TiledPlan tiled_plan_of(int64_t M, int Kp, int N, int bits, int KC, int CT, int seg_steps) {
  TiledPlan p;
  p.KS = 1;
  const int64_t wbytes = (int64_t)Kp * N * bits / 8;     // packed codes of the layer
  const int64_t mb64 = (M + 63) / 64;                            // 64-row blocks
  if (seg_steps != 4) {
    p.tile = 1;
  } else if (M <= 16) {
    p.tile = 7;
  } else if (M <= 32) {
    p.tile = 6;
  } else if (M <= 64) {
    p.tile = 5;
  } else if (M <= 512 && KC <= 32 && mb64 * wbytes <= (int64_t(128) << 20)) {
    p.tile = 5;       // short K, and every 64-row block's pass over the weights fits the MALL
  } else if (tiles_of(M, CT, 0) >= 192) {
    p.tile = 0;
  } else {
    p.tile = 4;
  }
  const int64_t t = tiles_of(M, CT, p.tile);
  if (p.tile == 5 && M > 64) p.KS = t >= 192 ? 1 : 2;
  else if (p.tile == 6 || p.tile == 7) p.KS = ceil_div(256, t);
  else if (p.tile == 3 || p.tile == 5) p.KS = ceil_div(448, t);
  else if (t < 150) p.KS = ceil_div(224, t);
  // one row slice of launch_tiled (x and y offsets below 2^31) must hold all M rows
  const int64_t row_slice = ((int64_t(1) << 31) - 1) / (2 * (int64_t)(Kp > N ? Kp : N)) / 256 * 256;
  if (p.KS > 1 && (M * (int64_t)N * 4 > (int64_t)INT32_MAX || M > row_slice)) p.KS = 1;
  if (p.KS > KC / 4) p.KS = KC / 4 > 1 ? KC / 4 : 1;     // at least four chunks per slice
  p.kcs = (KC + p.KS - 1) / p.KS;
  p.KS = (KC + p.kcs - 1) / p.kcs;
  if (p.tile == 5 && t * p.KS <= 256) p.tile = 8;       // same tiles and slices, twice the waves
  return p;
}

}  // namespace gq
