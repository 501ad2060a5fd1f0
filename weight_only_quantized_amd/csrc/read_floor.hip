// Device read floor: the time to read a call's packed bytes once, nothing else.
//
// "Formats and kernels: FP8, INT8, INT4, Marlin, Machete" (its opening section) prices a small-M call
// of a weight-only layer by the time to stream its packed weight bytes from memory.  This kernel
// measures what that stream costs on the device: every wave reads one contiguous 8 KB span with all
// eight 16-byte-per-lane loads in flight at once (the shape that read fastest on MI355X among the
// per-wave spans and workgroup sizes measured: 4-wave workgroups, 4-8 KB per wave), with the
// non-temporal hint, and folds the data into one word that is stored only if it equals a value the
// fold cannot produce for the callers' data -- so the loads cannot be removed.
#include <hip/hip_runtime.h>

#include "bufmem.h"
#include "internal.h"

namespace gq {

constexpr int kFloorLoads = 8;                 // 16-byte loads per lane, all in flight
constexpr int kFloorWaveBytes = kFloorLoads * 64 * 16;

__global__ void __launch_bounds__(256) read_floor_kernel(const uint8_t* __restrict__ p, uint64_t bytes,
                                                         uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const uint64_t wave = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const uint64_t base = wave * kFloorWaveBytes;
  // one resource per wave over its own span (spans past 2^31 bytes stay addressable)
  const uint64_t span = base < bytes ? (bytes - base < (uint64_t)kFloorWaveBytes ? bytes - base : kFloorWaveBytes) : 0;
  const rsrc_t r = make_rsrc(p + (base < bytes ? base : 0), (uint32_t)span);
  u32x4 v[kFloorLoads];
#pragma unroll
  for (int u = 0; u < kFloorLoads; ++u)
    v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(u * 1024 + lane * 16), 0u, kAuxStream);
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kFloorLoads; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  if (acc == 0x9E3779B9u && span == 0) sink[0] = acc;    // never true: span 0 reads zeros only
}

hipError_t launch_read_floor(const void* p, size_t bytes, uint32_t* sink, hipStream_t s) {
  const uint64_t waves = (bytes + kFloorWaveBytes - 1) / kFloorWaveBytes;
  const uint64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL(read_floor_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(p), (uint64_t)bytes, sink);
  return hipGetLastError();
}

}  // namespace gq
