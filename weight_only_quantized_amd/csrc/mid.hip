// Host launcher of the mid family (kernel and per-width dispatch: mid_impl.h), and the kernel that
// adds its split-K partial sums.
#include <hip/hip_runtime.h>

#include "mid_impl.h"
#include "skinny_impl.h"

namespace gq {

static inline size_t align256m(size_t b) { return (b + 255) / 256 * 256; }

bool skinny_one_launch(const gptq_layer* L, int64_t M) {
  return skinny_reads_x_from_l2(M, L->KC, L->CT, L->bits, L->seg_steps) ||
         skinny_mx_long(M, L->KC, L->CT, L->seg_steps, L->has_perm != 0) ||
         // (act-order layers: the skinny path sorts x into the workspace first, skinny_needs_xsorted)
         skinny_copy_plan(M, L->KC, L->CT, L->bits, L->seg_steps, false).ok;
}

int mid_slices(const gptq_layer* L, int64_t M) { return mid_plan(L, M).KS; }
int mid_slice_chunks(const gptq_layer* L, int64_t M) { return mid_plan(L, M).cpw; }

bool uses_mid(const gptq_layer* L, int64_t M) {
  return M > 0 && !x_fits_lds(M, L->Kp) && !skinny_one_launch(L, M) &&
         !skinny_m1_rule(M, L->KC, L->seg_steps, L->has_perm != 0);
}

size_t ws_mid_part_bytes(const gptq_layer* L, int64_t M) {
  if (!uses_mid(L, M)) return 0;
  const int64_t rows = M < mid_rows_per_pass(L) ? M : mid_rows_per_pass(L);
  const MidPlan p = mid_plan(L, rows);
  return p.KS > 1 ? align256m((size_t)p.KS * rows * L->N * 4) : 0;
}

// y[m, n] = round(sum over slices s in order of part[s, m, n] + bias[n]); four outputs per
// thread.  Slices are read eight at a time, all eight loads in flight together (indices past KS
// re-read the last slice and are masked out of the sum).
template <int XT>
__global__ void __launch_bounds__(256) mid_reduce_kernel(const float* __restrict__ part, uint16_t* __restrict__ y,
                                                         int64_t mn4, int64_t mn, int KS, int N, const void* bias,
                                                         int bias_kind) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= mn4) return;
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  if (bias) {
    const int n0 = (int)((4 * i) % N);          // N % 4 == 0: the four outputs share a row
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = bias_at(bias, bias_kind, n0 + e);
  }
  for (int k0 = 0; k0 < KS; k0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4*>(part + min(k0 + u, KS - 1) * mn + 4 * i);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u < KS) s += v[u];
  }
  uint32_t lo = (uint32_t)to_out<XT>(s[0]) | ((uint32_t)to_out<XT>(s[1]) << 16);
  uint32_t hi = (uint32_t)to_out<XT>(s[2]) | ((uint32_t)to_out<XT>(s[3]) << 16);
  *reinterpret_cast<u32x2*>(y + 4 * i) = u32x2{lo, hi};
}

// One pass over rows [r0, r0 + rows) of x and y (x already in sorted order, row stride ld).
static hipError_t mid_pass(const GemmCall& c, const uint16_t* x, int ld, float* part, int64_t r0, int64_t rows) {
  const gptq_layer* L = c.L;
  const MidPlan p = mid_plan(L, rows);
  MidArgs a;
  a.wq = L->wq;
  a.meta = L->meta;
  a.scale32 = L->scale32;
  a.x = x + r0 * ld;
  a.ld = ld;
  a.part = p.KS > 1 ? part : nullptr;
  a.y = reinterpret_cast<uint16_t*>(c.y) + r0 * L->N;
  a.M = (int)rows; a.K = L->K; a.N = L->N; a.KC = L->KC; a.CT = L->CT; a.G = L->G;
  a.scale_kind = L->scales_dtype;
  segment_divisor(L, &a.gmagic, &a.gshift);
  a.cpw = p.cpw;
  a.bias = c.bias;
  hipError_t e;
  switch (L->bits) {
    case 2: e = mid_b2(a, p, c.x_bf16, L->seg_steps, c.stream); break;
    case 3: e = mid_b3(a, p, c.x_bf16, L->seg_steps, c.stream); break;
    case 4: e = mid_b4(a, p, c.x_bf16, L->seg_steps, c.stream); break;
    case 5: e = mid_b5(a, p, c.x_bf16, L->seg_steps, c.stream); break;
    case 6: e = mid_b6(a, p, c.x_bf16, L->seg_steps, c.stream); break;
    case 7: e = mid_b7(a, p, c.x_bf16, L->seg_steps, c.stream); break;
    default: e = mid_b8(a, p, c.x_bf16, L->seg_steps, c.stream); break;
  }
  if (e != hipSuccess || p.KS == 1) return e;
  return launch_part_reduce(a.part, a.y, rows, L->N, p.KS, c.bias, L->scales_dtype, c.x_bf16, c.stream);
}

hipError_t launch_part_reduce(const float* part, uint16_t* y, int64_t rows, int N, int KS, const void* bias,
                              int bias_kind, int x_bf16, hipStream_t s) {
  const int64_t mn = rows * (int64_t)N, mn4 = mn / 4;     // N is a multiple of 32
  const unsigned blocks = (unsigned)((mn4 + 255) / 256);
  if (x_bf16)
    hipLaunchKernelGGL(mid_reduce_kernel<1>, dim3(blocks), dim3(256), 0, s, part, y, mn4, mn, KS, N, bias, bias_kind);
  else
    hipLaunchKernelGGL(mid_reduce_kernel<0>, dim3(blocks), dim3(256), 0, s, part, y, mn4, mn, KS, N, bias, bias_kind);
  return hipGetLastError();
}

hipError_t launch_mid(const GemmCall& c) {
  const gptq_layer* L = c.L;
  uint8_t* base = reinterpret_cast<uint8_t*>(c.ws);
  const uint16_t* x;
  int ld;
  if (L->has_perm) {
    hipError_t e = launch_prep(c, false);
    if (e != hipSuccess) return e;
    x = reinterpret_cast<const uint16_t*>(base);
    ld = L->Kp;
    base += ws_xsorted_bytes(L, c.M);
  } else {
    x = reinterpret_cast<const uint16_t*>(c.x);
    ld = L->K;
  }
  // passes run in stream order and share the partial-sum area
  const int64_t step = mid_rows_per_pass(L);
  for (int64_t r0 = 0; r0 < c.M; r0 += step) {
    const hipError_t e = mid_pass(c, x, ld, reinterpret_cast<float*>(base), r0, c.M - r0 < step ? c.M - r0 : step);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gq
