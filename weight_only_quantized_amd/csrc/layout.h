// Runtime (kernel-private) weight layout of the GPTQ linear layer on gfx950.
//
// The checkpoint layout ("GPTQ packed checkpoint (safetensors / torch)", sections "GptqLayer"
// and "Reader") packs 32/bits codes per int32 along the input dimension K, row-major over N.
// The kernels instead want every lane of a 64-wide wave to fetch, with one contiguous 16-byte
// load, exactly the codes that feed its B operand of v_mfma_f32_16x16x32_{f16,bf16}:
//
//   16x16x32 B operand (verified on the device): lane l holds column j = l % 16 and the eight
//   consecutive k = 8 * (l / 16) + e, e = 0..7, of a 32-deep K step.
//
// Units.  Columns are cut into tiles of 16 (CT = N / 16 tiles) and the load-time-sorted input
// dimension into chunks of 128 (KC = Kp / 128, Kp = K rounded up to 128; padded inputs have
// code 0 and are multiplied by x = 0).  One unit = one (tile, chunk) = 16 x 128 codes =
// 256 * bits bytes, stored tile-major: unit index = ct * KC + kc.  Inside a unit, lane l owns the
// 32 codes  i = 8 * t + e  (t = MFMA step 0..3, e = 0..7) at sorted k = 128 kc + 32 t + 8 (l/16) + e
// and column n = 16 ct + l % 16, held in WPL = bits 32-bit words.  Word order inside a unit:
// [part][lane][w] with parts of up to four words (8-bit: two parts), so each wave-wide load of a
// part is one contiguous 64 x 16 B (or x 8 B / x 12 B) block.
//
// Code placement inside a lane's words is chosen so that four codes come out as the four bytes
// of one register ("byte vector" BV_j holds codes 4j .. 4j+3 in bytes 0..3) with one shift and
// one mask, for 2-, 3- and 4-bit codes:
//   4-bit: code i = 8t + 4h + b  at word t, bit 8b + 4h            (BV_{2t+h} = (w_t >> 4h) & 0x0F0F0F0F)
//   2-bit: code i = 16u + 4h + b at word u, bit 8b + 2h            (BV_{4u+h} = (w_u >> 2h) & 0x03030303)
//   3-bit: code i < 24, i = 8u + 4h + b at word u, bit 8b + 3h      (BV_{2u+h} = (w_u >> 3h) & 0x07070707)
//          code 24 + b: bits 0-1 at word 0 bit 8b+6, bit 2 at word 1 bit 8b+6
//          code 28 + b: bit 0 at word 1 bit 8b+7, bits 1-2 at word 2 bit 8b+6
//          (the two spare bits of every byte of the three words carry the last eight codes)
//   8-bit: code i = 8t + 4h + c  at word 2t + h, byte {0, 2, 1, 3}[c]
//          ((w & 0x00FF00FF) holds codes c = 0, 1 in its two 16-bit halves, (w >> 8) & 0x00FF00FF
//          codes c = 2, 3)
//   5/6/7-bit (b bits, s = 8 - b spare bits per byte): code i < 4b at word i / 4, byte i % 4, its
//          low b bits (BV_j = w_j & mask for j < b); the s spare bits of byte position p of the
//          b words, taken word by word, form a stream of b * s bits that holds the s remaining
//          codes of that byte position, 4b + 4e + p for e = 0 .. s - 1, b bits each, low bits
//          first (a code's bits come from up to b words; 7-bit: one spare bit per word)
//
// Group metadata is re-tiled the same way, one 32-bit record per (tile, group, column):
//   meta[(ct * G + g) * 16 + j] = scale bits (fp16/bf16, bits 0-15; 0 for f32 scales)
//                                 | (zero - 1 mod 2^16) << 16
// (the GPTQ v1 stored field; an AWQ zero is stored as it is, so its 0 becomes 0xFFFF)
// plus, for f32 scales only, scale32[(ct * G + g) * 16 + j] = the f32 bits.  One record per lane
// per segment keeps the kernels' metadata loads unconditional and width-uniform.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define GQ_HD __host__ __device__ __forceinline__
#else
#define GQ_HD inline
#endif

namespace gq {

constexpr int kChunkK = 128;   // sorted-K chunk of one unit
constexpr int kTileN = 16;     // columns per tile
constexpr int kLanes = 64;
constexpr int kIpermMaxKp = 8192;   // 16-bit inverse permutation kept up to this padded K

GQ_HD int words_per_lane(int bits) { return bits; }
GQ_HD int64_t unit_words(int bits) { return (int64_t)kLanes * bits; }

// Word offset (within a unit) of lane `lane`'s word `w`: up to four words a lane, lane-major;
// wider codes in two parts, words 0-3 (lane-major, 4 words a lane) then words 4 .. bits - 1.
GQ_HD int unit_word_offset(int bits, int lane, int w) {
  if (bits <= 4) return lane * bits + w;
  const int part = w >> 2, pw = part == 0 ? 4 : bits - 4;
  return part * (kLanes * 4) + lane * pw + (w & 3);
}

// A piece of a code: `nb` bits of word `word` starting at bit `bit` hold code bits
// [cbit, cbit + nb).  Every code has at most kMaxPieces pieces (one or two up to 4 bits and for
// 8 bits; up to `bits` for the spare-bit codes of 5/6/7 bits).
struct Piece { int word, bit, nb, cbit; };
constexpr int kMaxPieces = 8;

GQ_HD int code_pieces(int bits, int i, Piece* p) {
  if (bits == 4) { int t = i >> 3, h = (i >> 2) & 1, b = i & 3; p[0] = {t, 8 * b + 4 * h, 4, 0}; return 1; }
  if (bits == 2) { int u = i >> 4, h = (i >> 2) & 3, b = i & 3; p[0] = {u, 8 * b + 2 * h, 2, 0}; return 1; }
  if (bits == 8) {
    int t = i >> 3, h = (i >> 2) & 1, c = i & 3;
    const int byte_of[4] = {0, 2, 1, 3};
    p[0] = {2 * t + h, 8 * byte_of[c], 8, 0};
    return 1;
  }
  if (bits >= 5) {
    if (i < 4 * bits) { p[0] = {i >> 2, 8 * (i & 3), bits, 0}; return 1; }
    const int x = i - 4 * bits, pos_byte = x & 3, e = x >> 2, sp = 8 - bits;
    int np = 0, pos = bits * e, cbit = 0;
    while (cbit < bits) {
      const int u = pos / sp, o = pos % sp, take = (sp - o < bits - cbit) ? sp - o : bits - cbit;
      p[np++] = {u, 8 * pos_byte + bits + o, take, cbit};
      pos += take;
      cbit += take;
    }
    return np;
  }
  // bits == 3
  if (i < 24) { int u = i >> 3, h = (i >> 2) & 1, b = i & 3; p[0] = {u, 8 * b + 3 * h, 3, 0}; return 1; }
  int b = i & 3;
  if (i < 28) { p[0] = {0, 8 * b + 6, 2, 0}; p[1] = {1, 8 * b + 6, 1, 2}; return 2; }
  p[0] = {1, 8 * b + 7, 1, 0}; p[1] = {2, 8 * b + 6, 2, 1}; return 2;
}

// Segment -> group map (a segment is a 128-input chunk or a 32-input step; d = segments per group):
// group = min(segment / d, G - 1), computed without a divide instruction.  shift = log2(d) when d is
// a power of two, else -1 with magic = ceil(2^32 / d); then segment / d = (segment * magic) >> 32,
// exact whenever segment * (magic * d - 2^32) < 2^32, which holds for segment < 2^32 / d.
GQ_HD int segment_shift(int64_t d) {
  for (int b = 0; b < 31; ++b)
    if (d == (int64_t(1) << b)) return b;
  return -1;
}
GQ_HD uint32_t segment_magic(int64_t d) {
  return segment_shift(d) >= 0 ? 0u : (uint32_t)(((int64_t(1) << 32) + d - 1) / d);
}
GQ_HD int group_of_segment(int si, uint32_t magic, int shift, int G) {
  const int g = shift >= 0 ? (si >> shift) : (int)(((uint64_t)(uint32_t)si * magic) >> 32);
  return g < G - 1 ? g : G - 1;
}
// The same with both forms computed and combined through a mask: the select above, on a
// wave-uniform value, is compiled into a branch, and a branch join inside chunk code that has loads
// in flight makes the wave wait for all of them.
GQ_HD int group_of_segment_nb(int si, uint32_t magic, int shift, int G) {
  const uint32_t by_shift = (uint32_t)si >> (shift & 31);
  const uint32_t by_magic = (uint32_t)(((uint64_t)(uint32_t)si * magic) >> 32);
  const uint32_t m = 0u - (uint32_t)(shift >= 0);
  const int g = (int)((by_shift & m) | (by_magic & ~m));
  return g < G - 1 ? g : G - 1;
}

// Sorted-K offset within the chunk, and column within the tile, of lane code i.
GQ_HD int code_k_in_chunk(int lane, int i) { return 32 * (i >> 3) + 8 * (lane >> 4) + (i & 7); }
GQ_HD int lane_col(int lane) { return lane & 15; }

}  // namespace gq
