// Host check of the runtime layout map (weight_only_quantized_amd/csrc/layout.h): for every bit
// width 2..8, the 32 codes of a lane must cover every bit of the lane's words exactly once, every
// lane word must land at a distinct offset inside its unit, and each part's words of a lane must
// be consecutive (one load); the division-free segment -> group map
// must equal integer division for every divisor and segment a layer can have.  Built with g++ by
// tests/test_boundary_cpu.py; prints "ok" on success.
#include <cstdio>
#include <set>
#include "layout.h"

int main() {
  const int widths[7] = {2, 3, 4, 5, 6, 7, 8};
  for (int bits : widths) {
    unsigned used[8] = {0};
    int code_bits = 0;
    for (int i = 0; i < 32; ++i) {
      gq::Piece p[gq::kMaxPieces];
      int np = gq::code_pieces(bits, i, p);
      int cb = 0;
      for (int k = 0; k < np; ++k) {
        if (p[k].word < 0 || p[k].word >= bits || p[k].bit < 0 || p[k].bit + p[k].nb > 32) { printf("range %d %d\n", bits, i); return 1; }
        if (p[k].cbit != cb) { printf("cbit order %d %d\n", bits, i); return 1; }
        unsigned m = (p[k].nb == 32 ? 0xFFFFFFFFu : ((1u << p[k].nb) - 1u)) << p[k].bit;
        if (used[p[k].word] & m) { printf("overlap bits=%d code=%d\n", bits, i); return 1; }
        used[p[k].word] |= m;
        cb += p[k].nb;
      }
      if (cb != bits) { printf("width %d %d\n", bits, i); return 1; }
      code_bits += cb;
    }
    for (int w = 0; w < bits; ++w) if (used[w] != 0xFFFFFFFFu) { printf("hole bits=%d word=%d %08x\n", bits, w, used[w]); return 1; }
    // every word of a part is read by one load of 1..4 consecutive words at the lane's base
    for (int lane = 0; lane < 64; ++lane)
      for (int w = 1; w < bits; ++w)
        if ((w & 3) != 0 && gq::unit_word_offset(bits, lane, w) != gq::unit_word_offset(bits, lane, w - 1) + 1) {
          printf("part not contiguous bits=%d lane=%d w=%d\n", bits, lane, w); return 1;
        }
    std::set<int> offs;
    for (int lane = 0; lane < 64; ++lane)
      for (int w = 0; w < bits; ++w) offs.insert(gq::unit_word_offset(bits, lane, w));
    if ((int)offs.size() != 64 * bits || *offs.begin() != 0 || *offs.rbegin() != 64 * bits - 1) { printf("offsets %d\n", bits); return 1; }
    // k positions: the 64 lanes x 32 codes cover the 16 columns x 128 inputs of a unit once
    std::set<int> kn;
    for (int lane = 0; lane < 64; ++lane)
      for (int i = 0; i < 32; ++i) kn.insert(gq::code_k_in_chunk(lane, i) * 16 + gq::lane_col(lane));
    if ((int)kn.size() != 2048) { printf("k/n cover %d\n", bits); return 1; }
  }
  // segment -> group map: d = segments per group (1 .. 4096, and 2^30 for one group), segments
  // below 2^15 (K <= 2^20 in 32-input steps), G groups
  for (long long d = 1; d <= 4096; ++d) {
    const int sh = gq::segment_shift(d);
    const unsigned mg = gq::segment_magic(d);
    const int G = (int)((32768 + d - 1) / d);
    for (int si = 0; si < 32768; ++si) {
      const long long want = si / d < G - 1 ? si / d : G - 1;
      if (gq::group_of_segment(si, mg, sh, G) != want) { printf("group map d=%lld si=%d\n", d, si); return 1; }
    }
  }
  {
    const long long d = 1LL << 30;
    if (gq::segment_shift(d) != 30) { printf("shift 2^30\n"); return 1; }
    for (int si = 0; si < 32768; ++si)
      if (gq::group_of_segment(si, gq::segment_magic(d), gq::segment_shift(d), 1) != 0) { printf("one group\n"); return 1; }
  }
  printf("ok\n");
  return 0;
}
