// Host check of the launch plans (weight_only_quantized_amd/csrc/plans.h).  Skinny family, over
// every row count up to 64, every chunk count up to 160 and a spread of column-tile counts: every
// form a rule picks must fit what its kernel assumes -- the LDS of one workgroup, the wave bound it
// was built for, whole 1 KB copy pieces, every wave holding at least one real chunk, and the part
// and chunk counts the kernels are instantiated with.  Mid kernel: an instantiated (row blocks,
// chunks per slice) pair, slices covering K exactly once, the slice's x within 64 KB of LDS.
// Tiled family, up to 65536 rows: a tile of the table, slices covering K exactly once with at
// least four chunks each when K is split, split partial sums addressable by 32-bit offsets, and a
// grid within the launch limit.  Built with g++ by tests/test_boundary_cpu.py; prints "ok" on
// success.
#include <cstdio>
#include <initializer_list>

#include "plans.h"

static int fail(const char* what, long M, int KC, int CT, int bits, int seg, int uns) {
  printf("%s: M=%ld KC=%d CT=%d bits=%d seg=%d unsorted=%d\n", what, M, KC, CT, bits, seg, uns);
  return 1;
}

int main() {
  const int cts[] = {1, 2, 3, 7, 8, 31, 32, 33, 64, 100, 255, 256, 257, 320, 384, 512, 640, 864, 896,
                     1023, 1024, 1280, 1536, 1728, 1792, 2048, 4096, 8192};
  long plans = 0, m1 = 0;
  for (long M = 0; M <= 64; ++M)
    for (int KC = 1; KC <= 160; ++KC)
      for (int CT : cts)
        for (int bits : {2, 3, 4, 8})
          for (int seg : {1, 4})
            for (int uns : {0, 1}) {
              const int Kp = KC * gq::kChunkK;
              const gq::CopyPlan p = gq::skinny_copy_plan(M, KC, CT, bits, seg, uns != 0);
              if (p.ok) {
                ++plans;
                const int W = p.mt == 2 ? 8 : 16;            // launch bound of the instantiation
                const long waves = (long)p.nks * p.cgs;
                const long Kxs = (long)p.nks * p.T * gq::kChunkK / p.ph;
                long lds = M * (Kxs + 8) * 2 + (Kxs / gq::kChunkK) * 16 * p.mt * 4;
                const long red = 16L * p.mt * 4 * 64 * 4;
                if (lds < red) lds = red;
                if (M < 2 || M > 32 || bits > 4 || seg != 4 || uns) return fail("form outside its rows, widths or groups", M, KC, CT, bits, seg, uns);
                if (p.mt != (M <= 16 ? 1 : 2)) return fail("row blocks", M, KC, CT, bits, seg, uns);
                if (p.T != 16 && p.T != 32) return fail("chunks per wave not built", M, KC, CT, bits, seg, uns);
                if (p.ph != 1 && p.ph != 2 && p.ph != 4) return fail("part count not built", M, KC, CT, bits, seg, uns);
                if (p.ph > 1 && p.T % (4 * p.ph) != 0) return fail("fewer than four chunks a part", M, KC, CT, bits, seg, uns);
                if ((long)p.nks * p.T < KC || (long)(p.nks - 1) * p.T >= KC) return fail("a wave without a real chunk", M, KC, CT, bits, seg, uns);
                if ((long)p.nks * p.T >= 2L * KC) return fail("more padding than chunks", M, KC, CT, bits, seg, uns);
                if (waves < 4 || waves > W || p.cgs < 1) return fail("waves a workgroup", M, KC, CT, bits, seg, uns);
                if (Kxs % 512 != 0) return fail("copy pieces", M, KC, CT, bits, seg, uns);
                if ((long)p.lds != lds || lds > 160 * 1024) return fail("LDS", M, KC, CT, bits, seg, uns);
              }
              if (gq::skinny_m1_rule(M, KC, seg, uns != 0)) {
                ++m1;
                const int T = gq::skinny_m1_chunks(KC);
                const int waves = (KC + T - 1) / T;
                if (M != 1 || seg != 4 || uns) return fail("M = 1 rule outside its case", M, KC, CT, bits, seg, uns);
                if (T != 4 && T != 8 && T != 16) return fail("M = 1 chunks per wave not built", M, KC, CT, bits, seg, uns);
                if (waves > 16 || (waves - 1) * T >= KC) return fail("M = 1 waves", M, KC, CT, bits, seg, uns);
                if ((long)(waves * T * gq::kChunkK + 8) * 2 + 16L * T * 4 > gq::kXLdsMax) return fail("M = 1 LDS", M, KC, CT, bits, seg, uns);
              }
              if (gq::skinny_m1_act_rule(M, Kp, seg, uns != 0)) {
                const int T = KC <= 32 ? 4 : (bits == 4 ? 16 : 8);   // the launcher's choice
                const int waves = (KC + T - 1) / T;
                if (M != 1 || seg != 4 || !uns || Kp > gq::kIpermMaxKp) return fail("act-order M = 1 rule outside its case", M, KC, CT, bits, seg, uns);
                if (waves > 8) return fail("act-order M = 1 waves", M, KC, CT, bits, seg, uns);
                if ((long)(waves * T * gq::kChunkK + 8) * 2 > gq::kXLdsMax) return fail("act-order M = 1 LDS", M, KC, CT, bits, seg, uns);
              }
              if (gq::x_fits_lds(M, Kp)) {
                if (M > 4 || (M + 1) * (long)(Kp + 8) * 2 > gq::kXLdsMax) return fail("staged x", M, KC, CT, bits, seg, uns);
              }
            }
  // mid kernel
  for (long M = 1; M <= 64; ++M)
    for (int KC = 1; KC <= 512; KC += (KC < 160 ? 1 : 7))
      for (int CT : cts)
        for (int seg : {1, 4}) {
          const gq::MidPlan p = gq::mid_plan_of(M, KC, CT, seg);
          const long rows = M < gq::mid_rows_per_pass_of(seg) ? M : gq::mid_rows_per_pass_of(seg);
          const bool built = seg == 4 ? ((p.MT == 1 && (p.cpw == 16 || p.cpw == 8 || p.cpw == 4)) ||
                                          (p.MT == 2 && (p.cpw == 8 || p.cpw == 4)) || (p.MT == 4 && p.cpw == 4))
                                       : (p.cpw == 4 && (p.MT == 1 || p.MT == 2));
          if (!built) return fail("mid: configuration not built", M, KC, CT, 0, seg, 0);
          if (16L * p.MT < rows || (p.MT > 1 && 16L * (p.MT / 2) >= rows)) return fail("mid: row blocks", M, KC, CT, 0, seg, 0);
          if ((long)p.KS * p.cpw < KC || (long)(p.KS - 1) * p.cpw >= KC) return fail("mid: slices", M, KC, CT, 0, seg, 0);
          if ((long)p.cpw * 16 * p.MT * 256 > 64 * 1024) return fail("mid: LDS", M, KC, CT, 0, seg, 0);
          if (p.KS > 65535) return fail("mid: grid", M, KC, CT, 0, seg, 0);
        }
  // tiled family
  const long tms[] = {1, 2, 16, 17, 33, 64, 65, 100, 128, 129, 256, 257, 512, 513, 768, 1024, 2048, 4096, 8192, 65536};
  const int tns[] = {32, 96, 256, 1024, 4096, 6144, 14336, 28672, 65536};
  for (long M : tms)
    for (int KC = 1; KC <= 512; KC += (KC < 40 ? 1 : 13))
      for (int N : tns)
        for (int bits : {2, 3, 4, 8})
          for (int seg : {1, 4}) {
            const int Kp = KC * gq::kChunkK, CT = N / 16;
            const gq::TiledPlan p = gq::tiled_plan_of(M, Kp, N, bits, KC, CT, seg);
            if (p.tile < 0 || p.tile >= gq::kNumTiles || (seg != 4 && p.tile != 1)) return fail("tiled: tile", M, KC, CT, bits, seg, 0);
            if (p.KS < 1 || p.kcs < 1 || (long)p.KS * p.kcs < KC || (long)(p.KS - 1) * p.kcs >= KC) return fail("tiled: slices", M, KC, CT, bits, seg, 0);
            if (p.KS > 1 && p.kcs < 4) return fail("tiled: slice shorter than four chunks", M, KC, CT, bits, seg, 0);
            if (p.KS > 1 && M * (long)N * 4 > 2147483647L) return fail("tiled: partial sums past 32-bit offsets", M, KC, CT, bits, seg, 0);
            const gq::TileShape& ts = gq::kTiles[p.tile];
            const long blocks = ((M + 16 * ts.WM - 1) / (16 * ts.WM)) * ((CT + ts.NW * ts.WN - 1) / (ts.NW * ts.WN)) * p.KS;
            if (blocks < 1 || blocks > 2147483647L) return fail("tiled: grid", M, KC, CT, bits, seg, 0);
          }
  if (plans == 0 || m1 == 0) { printf("no plans\n"); return 1; }
  printf("ok\n");
  return 0;
}
