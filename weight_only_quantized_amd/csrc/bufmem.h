// Buffer-resource loads (device only).
//
// A gfx9-family buffer resource lives in four scalar registers; a load then takes a per-lane
// 32-bit byte offset (VGPR), a wave-uniform byte offset (SGPR) and an immediate.  Streaming
// kernels keep each lane's offset fixed and advance only the scalar offset, so address
// arithmetic costs no vector ALU at all.  Offsets at or past the resource's byte size return
// zero without touching memory, which masks rows and tails without branches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dequant.h"

namespace gq {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

constexpr int kRsrcWord3 = 0x00020000;   // untyped (raw) buffer descriptor, gfx9 family
constexpr int kAuxStream = 2;            // nt: data read once, do not keep it in the caches
constexpr uint32_t kOob = 0x80000000u;   // a lane offset past every resource: loads return 0

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Wait until at most N vector-memory operations of this wave are outstanding (loads, and loads
// into LDS, complete in issue order); the other counters are left alone (s_waitcnt fields of
// gfx9: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// `words` consecutive 32-bit words at voff + soff of resource r.
template <int WORDS, int AUX>
__device__ __forceinline__ void load_words(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* out) {
  if constexpr (WORDS == 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  } else if constexpr (WORDS == 3) {
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, AUX);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2];
  } else if constexpr (WORDS == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
    out[0] = v[0]; out[1] = v[1];
  } else {
    out[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX);
  }
}

// A lane's `BITS` words of one unit (layout.h, unit_word_offset) at byte offset soff of resource
// r: one load of BITS words up to 4 bits; above, words 0-3 and then words 4 .. BITS - 1.  The two
// lane offsets come from unit_voff0 / unit_voff1, computed once per kernel.
template <int BITS>
__device__ __forceinline__ uint32_t unit_voff0(int lane) { return (uint32_t)lane * (BITS < 4 ? BITS : 4) * 4u; }
template <int BITS>
__device__ __forceinline__ uint32_t unit_voff1(int lane) {
  return BITS == 8 ? unit_voff0<BITS>(lane) + 1024u : 1024u + (uint32_t)lane * (BITS > 4 ? BITS - 4 : 0) * 4u;
}
template <int BITS, int AUX>
__device__ __forceinline__ void load_unit(rsrc_t r, uint32_t voff0, uint32_t voff1, uint32_t soff, uint32_t* out) {
  if constexpr (BITS <= 4) {
    load_words<BITS, AUX>(r, voff0, soff, out);
  } else {
    load_words<4, AUX>(r, voff0, soff, out);
    load_words<BITS - 4, AUX>(r, voff1, soff, out + 4);
  }
}

__device__ __forceinline__ u32x4 load_b128(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t load_b32(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
// Stores past the resource's byte size are dropped, like loads there return zero.
__device__ __forceinline__ void store_b16(rsrc_t r, uint16_t v, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, 0u, 0);
}
__device__ __forceinline__ void store_b32(rsrc_t r, uint32_t v, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, 0u, 0);
}

}  // namespace gq
