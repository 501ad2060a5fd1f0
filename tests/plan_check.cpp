// Host check of the skinny family's dispatch rules (weight_only_quantized_amd/csrc/skinny_plan.h):
// over every row count up to 64, every chunk count up to 160 and a spread of column-tile counts,
// every form a rule picks must fit what its kernel assumes -- the LDS of one workgroup, the wave
// bound it was built for, whole 1 KB copy pieces, every wave holding at least one real chunk, and
// the part counts and chunk counts the kernels are instantiated with.  Built with g++ by
// tests/test_boundary_cpu.py; prints "ok" on success.
#include <cstdio>
#include <initializer_list>

#include "skinny_plan.h"

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
  if (plans == 0 || m1 == 0) { printf("no plans\n"); return 1; }
  printf("ok\n");
  return 0;
}
