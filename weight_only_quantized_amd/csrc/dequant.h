// In-register dequantisation into v_mfma_f32_16x16x32_{f16,bf16} B operands (device only).
//
// The method ("39. Quantized checkpoints ...", "The format"; "GPTQ packed checkpoint", "Reader")
// computes W[n, k] = (code - zero) * scale.  "Formats and kernels: FP8, INT8, INT4, Marlin,
// Machete" (its INT4 -> fp16 conversion discussion) describes splicing an integer into the low
// mantissa bits of a float whose exponent makes one mantissa unit equal to 1, so that the bit
// pattern IS the float (magic + v) with no conversion instruction.  Re-targeted to gfx950:
//   * four codes come out of one register as its four bytes with one shift and one mask
//     (the byte vectors of layout.h);
//   * v_perm_b32 moves two bytes into the low bytes of two 16-bit halves and fills the high bytes
//     with 0x64 (fp16: 0x64vv = 1024 + v) or 0x43 (bf16: 0x43vv = 128 + v);
//   * fp16: one v_pk_add_f16 of -(1024 + zero) leaves code - zero EXACTLY in each half (8-bit
//     codes: the 16-bit halves of (w & 0x00FF00FF) | 0x64006400 hold 1024 + code, same add);
//   * bf16 (gfx950 has no packed bf16 add): the zero is subtracted in the integer domain first,
//     v = code + 16 - zero in [0, 30] per byte (one v_add_u32, no carries), so the operand is
//     144 + (code - zero) exactly, and the kernels remove the constant 144 with one extra term
//     -144 * sum_k x[m, k] per row and segment, fed in as the MFMA's initial accumulator;
//     5..8-bit bf16 codes go through fp32 (c - z is exact in bf16, no bias);
//   * the group scale multiplies each segment's fp32 partial sum (a group, or a 128-input chunk
//     of a larger group) -- it is never folded into the 16-bit operand, so no weight is rounded.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <int XT>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (XT == 0)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Bias of the B operand (144 for bf16 with 2/3/4-bit codes, else 0), and its negation as a
// bf16 pattern in both halves of a register (-144 = 0xC310).
template <int BITS, int XT> struct Bias { static constexpr bool any = false; static constexpr uint32_t neg2 = 0u; };
template <> struct Bias<2, 1> { static constexpr bool any = true; static constexpr uint32_t neg2 = 0xC310C310u; };
template <> struct Bias<3, 1> { static constexpr bool any = true; static constexpr uint32_t neg2 = 0xC310C310u; };
template <> struct Bias<4, 1> { static constexpr bool any = true; static constexpr uint32_t neg2 = 0xC310C310u; };

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Per-lane, per-segment zero term from the zero (0 .. 2^bits; zero_of).
template <int BITS, int XT>
__device__ __forceinline__ uint32_t zero_term(uint32_t zero) {
  if constexpr (XT == 0) return (0xE400u + zero) * 0x00010001u;            // fp16 -(1024 + zero), both halves
  else if constexpr (BITS <= 4) return (16u - zero) * 0x01010101u;         // + 16 - zero per byte
  else return zero;                                                        // the zero itself
}

// Byte vector j (codes 4j .. 4j+3 of the lane, see layout.h) from the lane's words.
template <int BITS>
__device__ __forceinline__ uint32_t byte_vector(const uint32_t* w, int j) {
  if constexpr (BITS == 4) return (w[j >> 1] >> (4 * (j & 1))) & 0x0F0F0F0Fu;
  else if constexpr (BITS == 2) return (w[j >> 2] >> (2 * (j & 3))) & 0x03030303u;
  else if constexpr (BITS == 3) {
    if (j < 6) return (w[j >> 1] >> (3 * (j & 1))) & 0x07070707u;
    const uint32_t comb = ((w[0] >> 6) & 0x03030303u) | ((w[1] >> 4) & 0x0C0C0C0Cu) | ((w[2] >> 2) & 0x30303030u);
    return j == 6 ? (comb & 0x07070707u) : ((comb >> 3) & 0x07070707u);
  } else {  // 5/6/7-bit: j < BITS in the low bits of word j's bytes, the rest from the spare bits
    static_assert(BITS >= 5 && BITS <= 7, "byte vectors of 2..7-bit codes");
    constexpr uint32_t ones = 0x01010101u;
    if (j < BITS) return w[j] & (ones * ((1u << BITS) - 1u));
    constexpr int sp = 8 - BITS;
    uint32_t r = 0;
    int pos = BITS * (j - BITS), cbit = 0;
#pragma unroll
    for (int q = 0; q < BITS; ++q) {      // at most BITS pieces, one per word
      if (cbit < BITS) {
        const int u = pos / sp, o = pos % sp, take = sp - o < BITS - cbit ? sp - o : BITS - cbit;
        r |= (w[u] >> (BITS + o - cbit)) & (ones * (((1u << take) - 1u) << cbit));
        pos += take;
        cbit += take;
      }
    }
    return r;
  }
}

__device__ __forceinline__ uint32_t pk_add_f16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) + __builtin_bit_cast(f16x2, b));
}

// B operand of MFMA step t (8 consecutive k of the lane's column): code - zero (fp16), or
// 144 + code - zero (bf16, 2/3/4-bit), or code - zero (bf16, 5..8-bit).
template <int BITS, int XT>
__device__ __forceinline__ u32x4 build_b(const uint32_t* w, int t, uint32_t zt) {
  u32x4 r;
  if constexpr (BITS >= 5 && BITS <= 7 && XT == 1) {
    // bf16 through fp32 (c - z is exact: |c - z| <= 128), bytes 0..3 of two byte vectors
    const float zf = (float)zt;
    const uint32_t bv[2] = {byte_vector<BITS>(w, 2 * t), byte_vector<BITS>(w, 2 * t + 1)};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t v = bv[p >> 1] >> (16 * (p & 1));     // bytes {0, 1} or {2, 3}
      const float lo = (float)(v & 0xFFu) - zf, hi2 = (float)((v >> 8) & 0xFFu) - zf;
      r[p] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi2) & 0xFFFF0000u);
    }
  } else if constexpr (BITS <= 7) {
    if constexpr (XT == 0) {
      const uint32_t b0 = byte_vector<BITS>(w, 2 * t), b1 = byte_vector<BITS>(w, 2 * t + 1);
      r[0] = pk_add_f16(__builtin_amdgcn_perm(0x64646464u, b0, 0x04010400u), zt);
      r[1] = pk_add_f16(__builtin_amdgcn_perm(0x64646464u, b0, 0x04030402u), zt);
      r[2] = pk_add_f16(__builtin_amdgcn_perm(0x64646464u, b1, 0x04010400u), zt);
      r[3] = pk_add_f16(__builtin_amdgcn_perm(0x64646464u, b1, 0x04030402u), zt);
    } else {
      const uint32_t b0 = byte_vector<BITS>(w, 2 * t) + zt;
      const uint32_t b1 = byte_vector<BITS>(w, 2 * t + 1) + zt;
      r[0] = __builtin_amdgcn_perm(0x43434343u, b0, 0x04010400u);
      r[1] = __builtin_amdgcn_perm(0x43434343u, b0, 0x04030402u);
      r[2] = __builtin_amdgcn_perm(0x43434343u, b1, 0x04010400u);
      r[3] = __builtin_amdgcn_perm(0x43434343u, b1, 0x04030402u);
    }
  } else if constexpr (XT == 0) {
    const uint32_t w0 = w[2 * t], w1 = w[2 * t + 1];
    r[0] = pk_add_f16((w0 & 0x00FF00FFu) | 0x64006400u, zt);
    r[1] = pk_add_f16(((w0 >> 8) & 0x00FF00FFu) | 0x64006400u, zt);
    r[2] = pk_add_f16((w1 & 0x00FF00FFu) | 0x64006400u, zt);
    r[3] = pk_add_f16(((w1 >> 8) & 0x00FF00FFu) | 0x64006400u, zt);
  } else {
    const float zf = (float)zt;
    const uint32_t ws[2] = {w[2 * t], w[2 * t + 1]};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t v = ws[p >> 1] >> (8 * (p & 1));      // bytes {0,2} or {1,3}
      const float lo = (float)(v & 0xFFu) - zf, hi2 = (float)((v >> 16) & 0xFFu) - zf;   // exact
      const uint32_t blo = __builtin_bit_cast(uint32_t, lo) >> 16, bhi = __builtin_bit_cast(uint32_t, hi2) >> 16;
      r[p] = blo | (bhi << 16);                            // exact: |c - z| <= 256 has <= 8 bits
    }
  }
  return r;
}

// B operand of MFMA step t without the zero: 1024 + code (fp16) or 128 + code (bf16, 2/3/4-bit
// codes), exact; the caller removes (offset + zero) * sum_k x[k] in fp32.
template <int BITS, int XT>
__device__ __forceinline__ u32x4 build_b_offset(const uint32_t* w, int t) {
  u32x4 r;
  if constexpr (BITS <= 4) {
    constexpr uint32_t hi = XT == 0 ? 0x64646464u : 0x43434343u;
    const uint32_t b0 = byte_vector<BITS>(w, 2 * t), b1 = byte_vector<BITS>(w, 2 * t + 1);
    r[0] = __builtin_amdgcn_perm(hi, b0, 0x04010400u);
    r[1] = __builtin_amdgcn_perm(hi, b0, 0x04030402u);
    r[2] = __builtin_amdgcn_perm(hi, b1, 0x04010400u);
    r[3] = __builtin_amdgcn_perm(hi, b1, 0x04030402u);
  } else {
    static_assert(XT == 0, "8-bit codes plus 128 do not fit bf16's significand");
    const uint32_t w0 = w[2 * t], w1 = w[2 * t + 1];
    r[0] = (w0 & 0x00FF00FFu) | 0x64006400u;
    r[1] = ((w0 >> 8) & 0x00FF00FFu) | 0x64006400u;
    r[2] = (w1 & 0x00FF00FFu) | 0x64006400u;
    r[3] = ((w1 >> 8) & 0x00FF00FFu) | 0x64006400u;
  }
  return r;
}

// Group scale of a metadata record (see layout.h); s32 holds the f32 bits when kind == 2.
// (Computed branch-free: a branch here would split the straight-line chunk code.)
__device__ __forceinline__ float scale_of(uint32_t rec, uint32_t s32, int kind) {
  const float f16v = (float)__builtin_bit_cast(_Float16, (uint16_t)(rec & 0xFFFFu));
  const float bf16v = __builtin_bit_cast(float, rec << 16);
  const float f32v = __builtin_bit_cast(float, s32);
  return kind == 0 ? f16v : (kind == 1 ? bf16v : f32v);
}
// The same picked through masks (no branch: see group_of_segment_nb), for chunk code with loads in
// flight.
__device__ __forceinline__ float scale_of_nb(uint32_t rec, uint32_t s32, int kind) {
  const uint32_t f16v = __builtin_bit_cast(uint32_t, (float)__builtin_bit_cast(_Float16, (uint16_t)(rec & 0xFFFFu)));
  const uint32_t bf16v = rec << 16;
  const uint32_t m1 = 0u - (uint32_t)(kind == 1), m2 = 0u - (uint32_t)(kind == 2);
  return __builtin_bit_cast(float, (((f16v & ~m1) | (bf16v & m1)) & ~m2) | (s32 & m2));
}
// The zero of a metadata record: its high half holds zero - 1 mod 2^16 (layout.h), which is the
// GPTQ v1 stored field as it is and 0xFFFF for an AWQ zero of 0.
__device__ __forceinline__ uint32_t zero_of(uint32_t rec) { return ((rec >> 16) + 1u) & 0xFFFFu; }

// Element n of an optional bias vector ("GPTQ packed checkpoint (safetensors / torch)", section
// "GptqLayer": same dtype as the scales), as fp32; 0 without one.  kind: 0 fp16, 1 bf16, 2 f32.
__device__ __forceinline__ float bias_at(const void* bias, int kind, int n) {
  if (!bias) return 0.f;
  if (kind == 2) return reinterpret_cast<const float*>(bias)[n];
  const uint16_t h = reinterpret_cast<const uint16_t*>(bias)[n];
  return kind == 0 ? (float)__builtin_bit_cast(_Float16, h) : __builtin_bit_cast(float, (uint32_t)h << 16);
}

template <int XT>
__device__ __forceinline__ uint16_t to_out(float v) {
  if constexpr (XT == 0) return __builtin_bit_cast(uint16_t, (_Float16)v);
  else return __builtin_bit_cast(uint16_t, (__bf16)v);
}

}  // namespace gq
