// GPTQ quantizer on the GPU: the step that produces a layer's codes, scales and zeros from its float
// weights and the Hessian of its calibration inputs.
//
// "39. Quantized checkpoints: GPTQ, AWQ, FP8, FP4 and trellis codes", section "GPTQ": H = 2 X^T X / n
// shared by every output row; never-active inputs get H_ii = 1 and zero weights; act-order visits
// inputs from the largest H_ii down; the damped H (damp times the mean diagonal on the diagonal) is
// inverted through Cholesky factorizations and the upper Cholesky factor U of H^-1 drives the
// error feedback: column i's error e = (w_i - quant(w_i)) / U_ii updates every later column j by
// -e U_ij, inside a block of 128 columns at once and beyond the block with one matrix product per
// block ("lazy batch updates"); a group's grid is taken from the current, already corrected
// weights when the loop enters it.  The page computes in float32; so does this file, with
// contraction off so that every rounding happens where the page's expressions put it.
//
// Design on gfx950: the output rows are independent given U, so the column loop of a block runs
// with one wave per row (lane l holds block columns l and l + 64, U's block in LDS, the current
// column broadcast across the wave); the Hessian is a float64-accumulated product of the inputs;
// the factorization (POTRF), the triangular inverse (TRTRI) and the per-block update GEMM are plain
// library calls
// (rocSOLVER / rocBLAS), loaded on first use so that the GEMM path does not depend on them.
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <dlfcn.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <numeric>
#include <vector>

#include "internal.h"

namespace gq {

constexpr int kQBlock = 128;   // the page's lazy-update block

// ---- Hessian: H[i, j] = 2 / S * sum_s x[s, i] x[s, j], float64 sums rounded once ----------------
// Workgroup tile 64 x 64 (16 x 16 threads of 4 x 4 outputs); 32 rows of x per LDS stage.
__global__ void __launch_bounds__(256) hessian_kernel(const void* __restrict__ x, int64_t S, int K, int xt,
                                                      float* __restrict__ H, double scale) {
  __shared__ double xa[32][64];
  __shared__ double xb[32][64];
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  double acc[4][4] = {};
  for (int64_t s0 = 0; s0 < S; s0 += 32) {
    for (int e = t; e < 32 * 64; e += 256) {
      const int r = e >> 6, c = e & 63;
      const int64_t s = s0 + r;
      double va = 0.0, vb = 0.0;
      if (s < S) {
        const int64_t ia = s * K + i0 + c, ib = s * K + j0 + c;
        if (xt == GPTQ_F32) {
          if (i0 + c < K) va = reinterpret_cast<const float*>(x)[ia];
          if (j0 + c < K) vb = reinterpret_cast<const float*>(x)[ib];
        } else {
          const uint16_t* xs = reinterpret_cast<const uint16_t*>(x);
          if (i0 + c < K) va = xt == GPTQ_F16 ? (double)__builtin_bit_cast(_Float16, xs[ia])
                                              : (double)__builtin_bit_cast(float, (uint32_t)xs[ia] << 16);
          if (j0 + c < K) vb = xt == GPTQ_F16 ? (double)__builtin_bit_cast(_Float16, xs[ib])
                                              : (double)__builtin_bit_cast(float, (uint32_t)xs[ib] << 16);
        }
      }
      xa[r][c] = va;
      xb[r][c] = vb;
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { a[u] = xa[r][ty * 4 + u]; b[u] = xb[r][tx * 4 + u]; }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] += a[u] * b[v];
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + ty * 4 + u, j = j0 + tx * 4 + v;
      if (i < K && j < K) H[(int64_t)i * K + j] = (float)(acc[u][v] * scale);
    }
}

// ---- set-up: diagonal, permuted and damped H, permuted W ------------------------------------------
__global__ void diag_kernel(const float* __restrict__ H, int K, float* __restrict__ d) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < K) d[i] = H[(int64_t)i * K + i];
}

// Hp[i, j] = H[p_i, p_j]; on the diagonal a never-active input reads 1, then the damping is added.
__global__ void permute_h_kernel(const float* __restrict__ H, const int32_t* __restrict__ perm,
                                 const uint8_t* __restrict__ dead, float damp_add, int K, float* __restrict__ Hp) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)K * K) return;
  const int i = (int)(e / K), j = (int)(e % K);
  float v = H[(int64_t)perm[i] * K + perm[j]];
  if (i == j) {
    if (dead[perm[i]]) v = 1.f;
    v = v + damp_add;
  }
  Hp[e] = v;
}

__global__ void permute_w_kernel(const float* __restrict__ W, const int32_t* __restrict__ perm,
                                 const uint8_t* __restrict__ dead, int N, int K, float* __restrict__ Wp) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)N * K) return;
  const int64_t n = e / K;
  const int c = (int)(e % K);
  Wp[e] = dead[perm[c]] ? 0.f : W[n * K + perm[c]];
}

// ---- the column loop of one block ----------------------------------------------------------------
// Wave w of the workgroup owns row n; lane l holds the block's columns l and l + 64 (w0, w1).  U's
// block [bw x bw] sits in LDS.  Group grids: when column col opens a group, the grid comes from the
// next gs columns' current values -- the block's corrected ones and, past the block, the row as the
// earlier blocks' updates left it -- min and max reduced across the wave, widened to contain 0.
// A block inside a longer group reads that group's grid back from scales / zeros.
template <int NW>
__global__ void __launch_bounds__(64 * NW) gptq_block_kernel(const float* __restrict__ Wp, const float* __restrict__ U,
                                                            uint8_t* __restrict__ cp, float* __restrict__ Err,
                                                            float* __restrict__ scales, int32_t* __restrict__ zeros,
                                                            int N, int K, int i1, int bw, int gs, int G, int bits) {
  __shared__ float Ub[kQBlock][kQBlock];
  for (int e = threadIdx.x; e < kQBlock * kQBlock; e += 64 * NW) {
    const int r = e >> 7, c = e & 127;
    Ub[r][c] = (r < bw && c < bw) ? U[(int64_t)(i1 + r) * K + i1 + c] : 0.f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * NW + (threadIdx.x >> 6);
  if (n >= N) return;                                  // no barrier follows
  const float* wrow = Wp + (int64_t)n * K;
  const int c0 = lane, c1 = lane + 64;
  float w0 = c0 < bw ? wrow[i1 + c0] : 0.f;
  float w1 = c1 < bw ? wrow[i1 + c1] : 0.f;
  float q0 = 0.f, q1 = 0.f, e0 = 0.f, e1 = 0.f;
  const float top = (float)((1 << bits) - 1);
  // a group opened by an earlier block (group_size above the block) keeps the grid it wrote
  float scale = 1.f, zero = 0.f;
  if (i1 % gs != 0) {
    scale = scales[(int64_t)n * G + i1 / gs];
    zero = (float)zeros[(int64_t)n * G + i1 / gs];
  }
  for (int i = 0; i < bw; ++i) {
    const int col = i1 + i;
    if (col % gs == 0) {
      const int end = min(col + gs, K);
      float mn = INFINITY, mx = -INFINITY;
      if (c0 >= i && c0 < bw && i1 + c0 < end) { mn = fminf(mn, w0); mx = fmaxf(mx, w0); }
      if (c1 >= i && c1 < bw && i1 + c1 < end) { mn = fminf(mn, w1); mx = fmaxf(mx, w1); }
      for (int c = i1 + bw + lane; c < end; c += 64) {
        const float v = wrow[c];
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
      }
      for (int o = 32; o > 0; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
      }
      const float lo = fminf(mn, 0.f), hi = fmaxf(mx, 0.f);
      if (hi == lo) {
        scale = 1.f;
        zero = 0.f;
      } else {
        scale = (hi - lo) / top;
        zero = rintf(-lo / scale);
      }
      if (lane == 0) {
        scales[(int64_t)n * G + col / gs] = scale;
        zeros[(int64_t)n * G + col / gs] = (int32_t)zero;
      }
    }
    const float wi = __shfl(i < 64 ? w0 : w1, i & 63);
    const float q = fminf(fmaxf(rintf(wi / scale + zero), 0.f), top);
    const float err = (wi - scale * (q - zero)) / Ub[i][i];
    if (c0 >= i && c0 < bw) w0 = w0 - err * Ub[i][c0];
    if (c1 >= i && c1 < bw) w1 = w1 - err * Ub[i][c1];
    if (lane == (i & 63)) {
      if (i < 64) { q0 = q; e0 = err; }
      else { q1 = q; e1 = err; }
    }
  }
  if (c0 < bw) {
    cp[(int64_t)n * K + i1 + c0] = (uint8_t)q0;
    Err[(int64_t)n * kQBlock + c0] = e0;
  }
  if (c1 < bw) {
    cp[(int64_t)n * K + i1 + c1] = (uint8_t)q1;
    Err[(int64_t)n * kQBlock + c1] = e1;
  }
}

// U from the inverse of the Cholesky factor of the reversed Hessian: with P = J Hp J = L L^T (J the
// order reversal) Hp = (J L J)(J L J)^T, so the upper factor of Hp^-1 is U = J L^-1 J -- the factor
// the page obtains from cholesky(cholesky_inverse(cholesky(Hp)), upper), with one factorization and
// one triangular inverse.  rocSOLVER leaves L^-1 column-major, i.e. mem[i][j] = L^-1[j][i] for
// j >= i row-major, and U[i][j] = L^-1[K-1-i][K-1-j] = mem[K-1-j][K-1-i]: an involution of the upper
// triangle, applied in place by swapping each pair once.
__global__ void reverse_upper_kernel(float* __restrict__ A, int K) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)K * K) return;
  const int i = (int)(e / K), j = (int)(e % K);
  if (j < i) return;
  const int pi = K - 1 - j, pj = K - 1 - i;
  const int64_t pe = (int64_t)pi * K + pj;
  if (e >= pe) return;                       // the pair's other element does the swap
  const float a = A[e], b = A[pe];
  A[e] = b;
  A[pe] = a;
}

// codes back in the original column order; g_idx of original column perm[c] is c / gs.
__global__ void unpermute_kernel(const uint8_t* __restrict__ cp, const int32_t* __restrict__ perm, int N, int K,
                                 int gs, uint8_t* __restrict__ codes, int32_t* __restrict__ g_idx) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)N * K) return;
  const int64_t n = e / K;
  const int c = (int)(e % K);
  codes[n * K + perm[c]] = cp[e];
  if (n == 0) g_idx[perm[c]] = c / gs;
}

// ---- checkpoint writer: logical codes / zeros / scales -> checkpoint tensors -----------------------
// "39. Quantized checkpoints ...", section "GPTQ" (the writer: codes along the input dimension, low
// bits first; zeros along the output dimension, stored minus one; scales [groups, out]), with the
// word rules of the repack side: continuous words (a 3-bit code may straddle two words of a
// 96-bit stream), or GPTQ_P planes (widths 2 | 2+1 | 4 | 4+1 | 4+2 | 4+2+1 | 8, low bits first).
// Packs the 32 values v[0..31] of one block into `bits` words w[0..bits-1].
__device__ __forceinline__ void pack_block32(const uint32_t* v, int bits, bool planar, uint32_t* w) {
  for (int i = 0; i < bits; ++i) w[i] = 0u;
  if (!planar) {
    for (int j = 0; j < 32; ++j) {
      const int bit = bits * j, wi = bit >> 5, sh = bit & 31;
      w[wi] |= v[j] << sh;
      if (sh + bits > 32) w[wi + 1] |= v[j] >> (32 - sh);
    }
    return;
  }
  int pw[3], np = 0;
  if (bits == 3) { pw[0] = 2; pw[1] = 1; np = 2; }
  else if (bits <= 4 || bits == 8) { pw[0] = bits; np = 1; }
  else { pw[0] = 4; pw[1] = bits == 5 ? 1 : 2; pw[2] = 1; np = bits == 7 ? 3 : 2; }
  int row = 0, low = 0;
  for (int p = 0; p < np; ++p) {
    const int per = 32 / pw[p];
    for (int j = 0; j < 32; ++j)
      w[row + j / per] |= ((v[j] >> low) & ((1u << pw[p]) - 1u)) << (pw[p] * (j % per));
    row += pw[p];
    low += pw[p];
  }
}

// qweight: thread per (block of 32 inputs kb, output n): codes[n, 32 kb .. 32 kb + 31].
__global__ void pack_codes_kernel(const uint8_t* __restrict__ codes, int N, int K, int bits, int planar,
                                  uint32_t* __restrict__ qweight) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)(K / 32) * N) return;
  const int n = (int)(t % N), kb = (int)(t / N);
  uint32_t v[32], w[8];
  for (int j = 0; j < 32; ++j) v[j] = codes[(int64_t)n * K + 32 * kb + j];
  pack_block32(v, bits, planar != 0, w);
  for (int i = 0; i < bits; ++i) qweight[(int64_t)(kb * bits + i) * N + n] = w[i];
}

// qzeros and scales: thread per (group g, block of 32 outputs nb); v1 stores zero - 1 (masked).
__global__ void pack_meta_kernel(const float* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int G,
                                 int bits, int planar, int minus_one, int sdt, uint32_t* __restrict__ qzeros,
                                 void* __restrict__ scales_out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)G * (N / 32)) return;
  const int g = (int)(t % G), nb = (int)(t / G);
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t v[32], w[8];
  for (int j = 0; j < 32; ++j) {
    const int n = 32 * nb + j;
    const uint32_t z = (uint32_t)zeros[(int64_t)n * G + g];
    v[j] = (minus_one ? z - 1u : z) & mask;
    const float sv = scales[(int64_t)n * G + g];
    const int64_t o = (int64_t)g * N + n;
    if (sdt == GPTQ_F32) {
      reinterpret_cast<float*>(scales_out)[o] = sv;
    } else if (sdt == GPTQ_F16) {
      reinterpret_cast<uint16_t*>(scales_out)[o] = __builtin_bit_cast(uint16_t, (_Float16)sv);
    } else {   // bf16, round to nearest even (scales are finite)
      const uint32_t u = __builtin_bit_cast(uint32_t, sv);
      reinterpret_cast<uint16_t*>(scales_out)[o] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    }
  }
  pack_block32(v, bits, planar != 0, w);
  const int zld = N / 32 * bits;
  for (int i = 0; i < bits; ++i) qzeros[(int64_t)g * zld + nb * bits + i] = w[i];
}

// ---- rocSOLVER / rocBLAS, loaded on first use -----------------------------------------------------
struct LinAlg {
  bool ok = false;
  rocblas_status (*create)(rocblas_handle*) = nullptr;
  rocblas_status (*destroy)(rocblas_handle) = nullptr;
  rocblas_status (*set_stream)(rocblas_handle, hipStream_t) = nullptr;
  rocblas_status (*sgemm)(rocblas_handle, rocblas_operation, rocblas_operation, rocblas_int, rocblas_int, rocblas_int,
                          const float*, const float*, rocblas_int, const float*, rocblas_int, const float*, float*,
                          rocblas_int) = nullptr;
  rocblas_status (*potrf)(rocblas_handle, rocblas_fill, rocblas_int, float*, rocblas_int, rocblas_int*) = nullptr;
  rocblas_status (*trtri)(rocblas_handle, rocblas_fill, rocblas_diagonal, rocblas_int, float*, rocblas_int,
                          rocblas_int*) = nullptr;
};

static const LinAlg& linalg() {
  static LinAlg L;
  static std::once_flag once;
  std::call_once(once, [] {
    void* blas = dlopen("librocblas.so.5", RTLD_NOW | RTLD_GLOBAL);
    if (!blas) blas = dlopen("/opt/rocm/lib/librocblas.so.5", RTLD_NOW | RTLD_GLOBAL);
    void* sol = dlopen("librocsolver.so.0", RTLD_NOW | RTLD_GLOBAL);
    if (!sol) sol = dlopen("/opt/rocm/lib/librocsolver.so.0", RTLD_NOW | RTLD_GLOBAL);
    if (!blas || !sol) return;
    L.create = (decltype(L.create))dlsym(blas, "rocblas_create_handle");
    L.destroy = (decltype(L.destroy))dlsym(blas, "rocblas_destroy_handle");
    L.set_stream = (decltype(L.set_stream))dlsym(blas, "rocblas_set_stream");
    L.sgemm = (decltype(L.sgemm))dlsym(blas, "rocblas_sgemm");
    L.potrf = (decltype(L.potrf))dlsym(sol, "rocsolver_spotrf");
    L.trtri = (decltype(L.trtri))dlsym(sol, "rocsolver_strtri");
    L.ok = L.create && L.destroy && L.set_stream && L.sgemm && L.potrf && L.trtri;
  });
  return L;
}

static inline size_t al256(size_t b) { return (b + 255) / 256 * 256; }

size_t quantize_workspace_bytes(int N, int K) {
  return al256((size_t)N * K * 4) + al256((size_t)K * K * 4) + al256((size_t)N * kQBlock * 4) + al256((size_t)N * K) +
         al256((size_t)K * 4) + al256((size_t)K * 4) + al256((size_t)K) + 256;
}

}  // namespace gq

using namespace gq;

extern "C" {

gptq_status gptq_hessian(const void* x, int64_t S, int32_t K, int32_t x_dtype, float* H, void* stream) {
  if (!x || !H || S <= 0 || K <= 0 || K > (1 << 15)) return GPTQ_E_INVALID_ARG;
  if (x_dtype != GPTQ_F16 && x_dtype != GPTQ_BF16 && x_dtype != GPTQ_F32) return GPTQ_E_INVALID_ARG;
  if (S * (int64_t)K > (int64_t(1) << 40)) return GPTQ_E_INVALID_ARG;
  const int tiles = (K + 63) / 64;
  hipLaunchKernelGGL(hessian_kernel, dim3(tiles, tiles), dim3(256), 0, (hipStream_t)stream, x, S, K, x_dtype, H,
                     2.0 / (double)S);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? GPTQ_OK : hip_fail(e);
}

gptq_status gptq_quantize_workspace_size(int32_t N, int32_t K, size_t* bytes) {
  if (!bytes || N <= 0 || K <= 0) return GPTQ_E_INVALID_ARG;
  *bytes = quantize_workspace_bytes(N, K);
  return GPTQ_OK;
}

gptq_status gptq_quantize(const float* W, const float* H, int32_t N, int32_t K, const gptq_quant_params* p,
                          uint8_t* codes, float* scales, int32_t* zeros, int32_t* g_idx, void* workspace,
                          size_t workspace_bytes, void* stream_) {
  if (!W || !H || !p || !codes || !scales || !zeros || !g_idx) return GPTQ_E_INVALID_ARG;
  if (p->reserved != 0 || !(p->damp >= 0.f) || p->damp > 1.f) return GPTQ_E_INVALID_ARG;
  if (p->bits < 2 || p->bits > 8) return GPTQ_E_UNSUPPORTED;
  if (p->group_size != -1 && (p->group_size <= 0 || p->group_size % 32 != 0)) return GPTQ_E_UNSUPPORTED;
  if (N <= 0 || K <= 0 || K % 32 != 0 || K > 16384 || N > (1 << 20) || (int64_t)N * K > (int64_t(1) << 31))
    return GPTQ_E_SHAPE;
  const size_t need = quantize_workspace_bytes(N, K);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256) return GPTQ_E_WORKSPACE;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  const LinAlg& la = linalg();
  if (!la.ok) return GPTQ_E_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream_;
  const int gs = p->group_size == -1 ? K : p->group_size;
  const int G = (K + gs - 1) / gs;

  uint8_t* base = reinterpret_cast<uint8_t*>(workspace);
  float* Wp = reinterpret_cast<float*>(base);              base += al256((size_t)N * K * 4);
  float* Hp = reinterpret_cast<float*>(base);              base += al256((size_t)K * K * 4);
  float* Err = reinterpret_cast<float*>(base);             base += al256((size_t)N * kQBlock * 4);
  uint8_t* cp = base;                                      base += al256((size_t)N * K);
  int32_t* perm_d = reinterpret_cast<int32_t*>(base);      base += al256((size_t)K * 4);
  float* diag_d = reinterpret_cast<float*>(base);          base += al256((size_t)K * 4);
  uint8_t* dead_d = base;                                  base += al256((size_t)K);
  rocblas_int* info_d = reinterpret_cast<rocblas_int*>(base);

  // diagonal -> host: never-active inputs, the visiting order and the damping term (O(K) set-up)
  hipLaunchKernelGGL(diag_kernel, dim3((K + 255) / 256), dim3(256), 0, s, H, K, diag_d);
  std::vector<float> d(K);
  e = hipMemcpyAsync(d.data(), diag_d, sizeof(float) * K, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  std::vector<uint8_t> dead(K);
  for (int i = 0; i < K; ++i) {
    dead[i] = d[i] == 0.f;
    if (dead[i]) d[i] = 1.f;
  }
  std::vector<int32_t> perm(K);
  std::iota(perm.begin(), perm.end(), 0);
  if (p->act_order) std::stable_sort(perm.begin(), perm.end(), [&](int a, int b) { return d[a] > d[b]; });
  std::vector<int32_t> rperm(perm.rbegin(), perm.rend());     // the reversed visiting order
  double sum = 0.0;
  for (int i = 0; i < K; ++i) sum += d[i];
  const float damp_add = p->damp * (float)(sum / K);
  e = hipMemcpyAsync(perm_d, rperm.data(), sizeof(int32_t) * K, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(dead_d, dead.data(), K, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);            // rperm is reused below
  if (e != hipSuccess) return hip_fail(e);
  const int64_t kk = (int64_t)K * K, nk = (int64_t)N * K;
  hipLaunchKernelGGL(permute_h_kernel, dim3((unsigned)((kk + 255) / 256)), dim3(256), 0, s, H, perm_d, dead_d,
                     damp_add, K, Hp);
  e = hipMemcpyAsync(perm_d, perm.data(), sizeof(int32_t) * K, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e);
  hipLaunchKernelGGL(permute_w_kernel, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, s, W, perm_d, dead_d, N, K,
                     Wp);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e);

  // U = upper Cholesky factor of Hp^-1 = J L^-1 J with L the Cholesky factor of the reversed Hp
  // (reverse_upper_kernel): one POTRF, one TRTRI, one in-place reversal.
  rocblas_handle hb = nullptr;
  if (la.create(&hb) != rocblas_status_success) return GPTQ_E_UNSUPPORTED;
  gptq_status st = GPTQ_OK;
  rocblas_int info[2] = {0, 0};
  if (la.set_stream(hb, s) != rocblas_status_success ||
      la.potrf(hb, rocblas_fill_lower, K, Hp, K, info_d) != rocblas_status_success ||
      hipMemcpyAsync(&info[0], info_d, sizeof(rocblas_int), hipMemcpyDeviceToHost, s) != hipSuccess ||
      la.trtri(hb, rocblas_fill_lower, rocblas_diagonal_non_unit, K, Hp, K, info_d) != rocblas_status_success ||
      hipMemcpyAsync(&info[1], info_d, sizeof(rocblas_int), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    st = GPTQ_E_HIP;
  } else if (info[0] || info[1]) {
    st = GPTQ_E_NUMERIC;                       // not positive definite even after damping
  } else {
    hipLaunchKernelGGL(reverse_upper_kernel, dim3((unsigned)((kk + 255) / 256)), dim3(256), 0, s, Hp, K);
    if (hipGetLastError() != hipSuccess) st = GPTQ_E_HIP;
  }
  const float minus_one = -1.f, one = 1.f;
  for (int i1 = 0; st == GPTQ_OK && i1 < K; i1 += kQBlock) {
    const int bw = std::min(kQBlock, K - i1);
    // sixteen rows per workgroup share one 64 KB copy of U's block, so a compute unit keeps eight
    // waves per SIMD in flight (four rows per workgroup left it two, and each step's dependent
    // chain of broadcast, divisions and update exposed its latency)
    hipLaunchKernelGGL(gptq_block_kernel<16>, dim3((unsigned)((N + 15) / 16)), dim3(1024), 0, s, Wp, Hp, cp, Err,
                       scales, zeros, N, K, i1, bw, gs, G, p->bits);
    if (hipGetLastError() != hipSuccess) { st = GPTQ_E_HIP; break; }
    const int i2 = i1 + bw, R = K - i2;
    if (R > 0 && la.sgemm(hb, rocblas_operation_none, rocblas_operation_none, R, N, bw, &minus_one,
                          Hp + (int64_t)i1 * K + i2, K, Err, kQBlock, &one, Wp + i2, K) != rocblas_status_success)
      st = GPTQ_E_HIP;
  }
  if (st == GPTQ_OK) {
    hipLaunchKernelGGL(unpermute_kernel, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, s, cp, perm_d, N, K, gs,
                       codes, g_idx);
    if (hipGetLastError() != hipSuccess) st = GPTQ_E_HIP;
  }
  if (hipStreamSynchronize(s) != hipSuccess && st == GPTQ_OK) st = GPTQ_E_HIP;
  la.destroy(hb);
  return st;
}

gptq_status gptq_pack(const uint8_t* codes, const float* scales, const int32_t* zeros, int32_t N, int32_t K,
                      int32_t bits, int32_t group_size, int32_t checkpoint_format, int32_t scales_dtype,
                      int32_t* qweight, int32_t* qzeros, void* scales_out, void* stream) {
  if (!codes || !scales || !zeros || !qweight || !qzeros || !scales_out) return GPTQ_E_INVALID_ARG;
  const int f = checkpoint_format;
  if (f != GPTQ_FORMAT_GPTQ && f != GPTQ_FORMAT_GPTQ_V2 && f != GPTQ_FORMAT_GPTQ_P) return GPTQ_E_UNSUPPORTED;
  const bool planar = f == GPTQ_FORMAT_GPTQ_P;
  if (planar ? (bits < 2 || bits > 8) : (bits != 2 && bits != 3 && bits != 4 && bits != 8)) return GPTQ_E_UNSUPPORTED;
  if (group_size != -1 && (group_size <= 0 || group_size % 32 != 0)) return GPTQ_E_UNSUPPORTED;
  if (scales_dtype != GPTQ_F16 && scales_dtype != GPTQ_BF16 && scales_dtype != GPTQ_F32) return GPTQ_E_INVALID_ARG;
  if (N <= 0 || K <= 0 || N % 32 || K % 32 || N > (1 << 20) || K > (1 << 20) || (int64_t)N * K > (int64_t(1) << 36))
    return GPTQ_E_SHAPE;
  const int gs = group_size == -1 ? K : group_size;
  const int G = (K + gs - 1) / gs;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nw = (int64_t)(K / 32) * N, nm = (int64_t)G * (N / 32);
  hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, codes, N, K, bits,
                     planar ? 1 : 0, reinterpret_cast<uint32_t*>(qweight));
  hipLaunchKernelGGL(pack_meta_kernel, dim3((unsigned)((nm + 255) / 256)), dim3(256), 0, s, scales, zeros, N, G, bits,
                     planar ? 1 : 0, f == GPTQ_FORMAT_GPTQ_V2 ? 0 : 1, scales_dtype,
                     reinterpret_cast<uint32_t*>(qzeros), scales_out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? GPTQ_OK : hip_fail(e);
}

}  // extern "C"
