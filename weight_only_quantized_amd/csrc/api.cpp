// Host side of the C ABI: validation, handle lifecycle, dispatch and the decode test hook.
//
// Validation follows "GPTQ packed checkpoint (safetensors / torch)", section "Reject the file
// when" (GPTQ-001 .. GPTQ-006), with the load-time sort of the inputs by g_idx from
// "39. Quantized checkpoints: GPTQ, AWQ, FP8, FP4 and trellis codes", section "The format".
// Caller-supplied scratch is checked for capacity and alignment and never silently replaced,
// as "Kernel Backends Reference", section "Marlin and caller-owned scratch", asks of a scratch
// contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>
#include <vector>

#include "bank_spread.h"
#include "internal.h"

namespace gq {

static thread_local int32_t t_last_hip = 0;

gptq_status hip_fail(hipError_t e) {
  t_last_hip = (int32_t)e;
  return GPTQ_E_HIP;
}

static int groups_of(int K, int gs) { return gs == -1 ? 1 : (K + gs - 1) / gs; }

// MFMA K steps (of 32 inputs) per scale-fixup segment: a whole 128-input chunk when groups are
// whole chunks (group_size a multiple of 128, or -1: one group), else one step.
static int seg_steps_of(int gs_eff, int gs) {
  if (gs == -1) return 4;                 // one group: any segmentation of K is exact
  return (gs_eff / 32) % 4 == 0 ? 4 : 1;
}

static bool is_gfx950_device(int dev) {
  static std::mutex mu;
  static int cache[64];
  static bool init = false;
  std::lock_guard<std::mutex> g(mu);
  if (!init) { for (int i = 0; i < 64; ++i) cache[i] = -1; init = true; }
  if (dev < 0 || dev >= 64) return false;
  if (cache[dev] < 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return false;
    cache[dev] = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  }
  return cache[dev] == 1;
}

// Shape/format checks that need no g_idx values.
static RepackSource repack_source(int32_t format) {
  switch (format) {
    case GPTQ_FORMAT_AWQ_GEMM: return kSrcAwqGemm;
    case GPTQ_FORMAT_GPTQ_V2: return kSrcGptqV2;
    case GPTQ_FORMAT_GPTQ_P: return kSrcGptqPlanar;
    default: return kSrcGptq;
  }
}

static gptq_status validate_desc(const gptq_layer_desc* d) {
  if (!d || d->reserved != 0) return GPTQ_E_INVALID_ARG;
  const int b = d->bits, f = d->checkpoint_format;
  const bool awq = f == GPTQ_FORMAT_AWQ_GEMM, planar = f == GPTQ_FORMAT_GPTQ_P;
  if (f != GPTQ_FORMAT_GPTQ && f != GPTQ_FORMAT_GPTQ_V2 && !awq && !planar) return GPTQ_E_UNSUPPORTED;  // GPTQ-005
  if (planar ? (b < 2 || b > 8) : (b != 2 && b != 3 && b != 4 && b != 8)) return GPTQ_E_UNSUPPORTED;  // GPTQ-001
  if (awq && (b != 4 || d->desc_act)) return GPTQ_E_UNSUPPORTED;                // 4-bit, sequential groups
  if (d->scales_dtype != GPTQ_F16 && d->scales_dtype != GPTQ_BF16 && d->scales_dtype != GPTQ_F32)
    return GPTQ_E_INVALID_ARG;
  const int gs = d->group_size;
  if (gs != -1 && (gs <= 0 || gs % 32 != 0)) return GPTQ_E_UNSUPPORTED;
  const int64_t K = d->in_features, N = d->out_features;
  if (K <= 0 || K % 32 != 0 || K > (1 << 20)) return GPTQ_E_SHAPE;               // GPTQ-002
  if (N <= 0 || N % 32 != 0 || N > (1 << 20) || K * N > (int64_t(1) << 36)) return GPTQ_E_SHAPE;
  const int64_t G = groups_of((int)K, gs);
  if (awq) {
    if (d->qweight_shape[0] != K || d->qweight_shape[1] != N / 8) return GPTQ_E_SHAPE;
    if (d->qzeros_shape[0] != G || d->qzeros_shape[1] != N / 8) return GPTQ_E_SHAPE;
    if (d->g_idx_len != 0) return GPTQ_E_GIDX;                                   // no g_idx in AWQ
  } else {
    if (d->qweight_shape[0] != K / 32 * b || d->qweight_shape[1] != N) return GPTQ_E_SHAPE;
    if (d->qzeros_shape[0] != G || d->qzeros_shape[1] != N / 32 * b) return GPTQ_E_SHAPE;  // GPTQ-003
    if (d->g_idx_len != 0 && d->g_idx_len != K) return GPTQ_E_GIDX;               // GPTQ-004
  }
  if (d->scales_shape[0] != G || d->scales_shape[1] != N) return GPTQ_E_SHAPE;
  return GPTQ_OK;
}

// GPTQ-004 range check, the whole-group reading, and the stable sort (counting sort by group).
// perm (size K) receives the input index at each sorted position.
static gptq_status check_gidx_and_sort(const gptq_layer_desc* d, const int32_t* g, int32_t* perm,
                                       int* has_perm) {
  const int K = d->in_features;
  const int G = groups_of(K, d->group_size);
  const int gs_eff = d->group_size == -1 ? K : d->group_size;
  std::vector<int32_t> count(G + 1, 0);
  for (int k = 0; k < K; ++k) {
    if (g[k] < 0 || g[k] >= G) return GPTQ_E_GIDX;
    count[g[k] + 1]++;
  }
  // whole groups: group q must hold exactly the sorted positions [q*gs, min((q+1)*gs, K))
  for (int q = 0; q < G; ++q) {
    int want = (q + 1) * gs_eff < K ? gs_eff : K - q * gs_eff;
    if (count[q + 1] != want) return GPTQ_E_UNSUPPORTED;
  }
  for (int q = 0; q < G; ++q) count[q + 1] += count[q];
  int hp = 0;
  for (int k = 0; k < K; ++k) {
    int pos = count[g[k]]++;
    if (perm) perm[pos] = k;
    if (pos != k) hp = 1;
  }
  if (has_perm) *has_perm = hp;
  return GPTQ_OK;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// (the within-group order of act-order layers: bank_spread.h)

static void free_layer(gptq_layer* L) {
  if (!L) return;
  if (L->wq) (void)hipFree(L->wq);
  if (L->meta) (void)hipFree(L->meta);
  if (L->scale32) (void)hipFree(L->scale32);
  if (L->perm) (void)hipFree(L->perm);
  if (L->iperm) (void)hipFree(L->iperm);
  delete L;
}

// Live handles: every handle gptq_repack returned and gptq_destroy has not yet taken back.  A
// handle is checked by membership, so a destroyed (or never issued) pointer is refused without
// reading the memory it points to.
static std::mutex g_live_mu;
static std::unordered_set<const gptq_layer*>& live_handles() {
  static std::unordered_set<const gptq_layer*> s;
  return s;
}
static void register_handle(const gptq_layer* L) {
  std::lock_guard<std::mutex> g(g_live_mu);
  live_handles().insert(L);
}
// Removes h from the live set; false if it was not there.
static bool retire_handle(const gptq_layer* L) {
  std::lock_guard<std::mutex> g(g_live_mu);
  return live_handles().erase(L) == 1;
}

static gptq_status check_handle(gptq_handle_t h) {
  if (!h) return GPTQ_E_INVALID_ARG;
  std::lock_guard<std::mutex> g(g_live_mu);
  return live_handles().count(h) ? GPTQ_OK : GPTQ_E_INVALID_ARG;
}

// Library-owned scratch of gptq_gemm_noalloc, one copy per device for the life of the process.  In
// host code `scratch` is only the host-side stand-in of the symbol: its device address (different on
// every device) comes from hipGetSymbolAddress, taken once per device with that device current and
// kept in g_scratch_dev, and only that address is ever handed to kernels.
constexpr size_t kScratchBytes = GPTQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices];

// Device address of the current device's scratch (dev is the current device).
static gptq_status scratch_of_device(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return GPTQ_E_DEVICE;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p || !aligned(p, 256)) return GPTQ_E_HIP;
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return GPTQ_OK;
}

}  // namespace gq

using namespace gq;

extern "C" {

gptq_status gptq_validate(const gptq_layer_desc* desc, const int32_t* g_idx_host) {
  gptq_status s = validate_desc(desc);
  if (s != GPTQ_OK || !g_idx_host) return s;
  if (desc->g_idx_len != desc->in_features) return GPTQ_E_GIDX;
  return check_gidx_and_sort(desc, g_idx_host, nullptr, nullptr);
}

gptq_status gptq_repack(const gptq_layer_desc* desc, const int32_t* qweight, const int32_t* qzeros,
                        const void* scales, const int32_t* g_idx, void* stream_, gptq_handle_t* out) {
  if (!out) return GPTQ_E_INVALID_ARG;
  *out = nullptr;
  gptq_status st = validate_desc(desc);
  if (st != GPTQ_OK) return st;
  if (!qweight || !qzeros || !scales) return GPTQ_E_INVALID_ARG;
  if (!aligned(qweight, 4) || !aligned(qzeros, 4) || !aligned(scales, 4)) return GPTQ_E_INVALID_ARG;
  if (g_idx && desc->g_idx_len != desc->in_features) return GPTQ_E_GIDX;
  if (!g_idx && desc->g_idx_len != 0) return GPTQ_E_INVALID_ARG;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (!is_gfx950_device(dev)) return GPTQ_E_DEVICE;
  hipStream_t s = (hipStream_t)stream_;

  const int K = desc->in_features, N = desc->out_features;
  const int Kp = (K + kChunkK - 1) / kChunkK * kChunkK;
  std::vector<int32_t> perm_host(Kp, -1);
  int has_perm = 0;
  if (g_idx) {
    std::vector<int32_t> gh(K);
    e = hipMemcpyAsync(gh.data(), g_idx, sizeof(int32_t) * K, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e);
    st = check_gidx_and_sort(desc, gh.data(), perm_host.data(), &has_perm);
    if (st != GPTQ_OK) return st;
    if (has_perm) (void)spread_scatter_banks(K, Kp, desc->group_size == -1 ? K : desc->group_size, perm_host.data());
  } else {
    for (int k = 0; k < K; ++k) perm_host[k] = k;
  }

  gptq_layer* L = new (std::nothrow) gptq_layer();
  if (!L) return GPTQ_E_OOM;
  std::memset(L, 0, sizeof(*L));
  L->device = dev;
  L->K = K; L->N = N; L->group_size = desc->group_size;
  L->ckpt_bits = desc->bits;
  L->bits = desc->bits;   // 2..8-bit runtime widths (layout.h)
  L->gs_eff = desc->group_size == -1 ? K : desc->group_size;
  L->G = groups_of(K, desc->group_size);
  L->Kp = Kp; L->KC = Kp / kChunkK; L->CT = N / kTileN;
  L->scales_dtype = desc->scales_dtype;
  L->has_perm = has_perm;
  L->seg_steps = seg_steps_of(L->gs_eff, desc->group_size);

  const size_t wq_bytes = (size_t)L->CT * L->KC * unit_words(L->bits) * 4;
  const size_t meta_n = (size_t)L->CT * L->G * kTileN;
  const size_t s32_bytes = L->scales_dtype == GPTQ_F32 ? meta_n * 4 : 0;
  const size_t perm_bytes = sizeof(int32_t) * Kp;
  if (hipMalloc((void**)&L->wq, wq_bytes) != hipSuccess ||
      hipMalloc((void**)&L->meta, meta_n * 4) != hipSuccess ||
      (s32_bytes && hipMalloc((void**)&L->scale32, s32_bytes) != hipSuccess) ||
      hipMalloc((void**)&L->perm, perm_bytes) != hipSuccess) {
    (void)hipGetLastError();
    free_layer(L);
    return GPTQ_E_OOM;
  }
  L->bytes = (int64_t)(wq_bytes + meta_n * 4 + s32_bytes + (has_perm ? perm_bytes : 0));
  e = hipMemcpyAsync(L->perm, perm_host.data(), perm_bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = launch_repack(L, qweight, qzeros, scales, repack_source(desc->checkpoint_format), s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    free_layer(L);
    return hip_fail(e);
  }
  if (!has_perm) {  // identity order: the kernels do not need the tables
    (void)hipFree(L->perm);
    L->perm = nullptr;
  } else if (Kp <= kIpermMaxKp) {
    // 16-bit sorted positions for the kernels that scatter x through them (the skinny kernel's
    // LDS staging of a whole row, where they halve the bytes every workgroup reads before its
    // first chunk, and the prep's sorted copy); Kp <= 8192
    std::vector<uint16_t> ip(K);
    for (int j = 0; j < Kp; ++j)
      if (perm_host[j] >= 0) ip[perm_host[j]] = (uint16_t)j;
    if (hipMalloc((void**)&L->iperm, sizeof(uint16_t) * K) != hipSuccess) {
      (void)hipGetLastError();
      free_layer(L);
      return GPTQ_E_OOM;
    }
    e = hipMemcpy(L->iperm, ip.data(), sizeof(uint16_t) * K, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      free_layer(L);
      return hip_fail(e);
    }
    L->bytes += (int64_t)sizeof(uint16_t) * K;
  }
  register_handle(L);
  *out = L;
  return GPTQ_OK;
}

// PATH_AUTO: the skinny family (skinny kernel, or the mid kernel's split K) up to 8 rows; from 9
// to 32 rows the skinny kernel where one of its one-launch forms takes the call (x read from L2,
// or the workgroup's copy of x in LDS: skinny_one_launch), else the tiled
// family when its K slices are long (8 chunks or more) while the mid kernel would cut K into more
// than 4 slices shorter than 16 chunks (of 4 chunks up to 16 rows), else the mid kernel; the tiled
// family (split K up to ~450 workgroups) above 32 rows.  Measured on MI355X with 4-bit g128 layers, fp16 x, mid vs tiled (two chunks in flight):
// 14336 x 4096, M = 8 / 16 / 24 / 32: 15.1 / 17.3 / 21.7 / 22.6 vs 17.2 / 16.0 / 16.8 / 17.6 us
// (tiled slices of 8 chunks, mid slices 28); 4096 x 6144, M = 24 / 32: 11.9 / 12.8 vs 12.3 / 13.7
// (tiled slices of 4); 8192 x 28672, M = 16 / 32: 33.7 / 45.9 vs 39.3 / 42.5 (tiled slices of 32,
// mid slices 4 at 16 rows, 8 at 32); 28672 x 8192, M = 12 / 16: 32.2 / 33.2 vs 38.0 / 38.4 (mid
// slices of 16 chunks); 5120 x 13824, M = 12 / 16: 15.1 / 15.9 vs 20.4 / 20.9 (mid slices of 8).
// At 48 rows and above the tiled family won on every shape measured.
static int32_t auto_path(const gptq_layer* L, int64_t M) {
  if (M <= 8) return GPTQ_PATH_SKINNY;
  if (M <= 32) {
    if (skinny_one_launch(L, M)) return GPTQ_PATH_SKINNY;
    // up to 16 rows only 4-chunk mid slices lose; from 17 rows any shorter than 16 chunks
    const int mid_cpw = mid_slice_chunks(L, M);
    return (tiled_slice_chunks(L, M) >= 8 && mid_slices(L, M) > 4 && (M > 16 ? mid_cpw < 16 : mid_cpw <= 4))
               ? GPTQ_PATH_TILED : GPTQ_PATH_SKINNY;
  }
  return GPTQ_PATH_TILED;
}

gptq_status gptq_workspace_size(gptq_handle_t h, int64_t M, int32_t x_dtype, int32_t path,
                                size_t* bytes) {
  gptq_status st = check_handle(h);
  if (st != GPTQ_OK) return st;
  if (!bytes || M < 0 || (x_dtype != GPTQ_F16 && x_dtype != GPTQ_BF16)) return GPTQ_E_INVALID_ARG;
  if (path == GPTQ_PATH_AUTO) path = auto_path(h, M);
  if (path != GPTQ_PATH_SKINNY && path != GPTQ_PATH_TILED) return GPTQ_E_INVALID_ARG;
  if (path == GPTQ_PATH_SKINNY && M > kSkinnyMaxM) return GPTQ_E_INVALID_ARG;
  size_t b = 0;
  if (M > 0) {
    const int bf16 = x_dtype == GPTQ_BF16;
    if (path == GPTQ_PATH_TILED) {
      if (tiled_needs_xsorted(h, bf16)) b += ws_xsorted_bytes(h, M);
      if (bf16) b += ws_rowexp_bytes(M);
      b += ws_tiled_part_bytes(h, M);
    } else {
      if (skinny_needs_xsorted(h, M)) b += ws_xsorted_bytes(h, M);
      b += ws_mid_part_bytes(h, M);
    }
  }
  *bytes = b;
  return GPTQ_OK;
}

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

static gptq_status gemm_impl(gptq_handle_t h, const void* x, int64_t M, int32_t x_dtype, const void* bias, void* y,
                             void* workspace, size_t workspace_bytes, int32_t path, void* stream) {
  gptq_status st = check_handle(h);
  if (st != GPTQ_OK) return st;
  if (M < 0 || M > (int64_t(1) << 24)) return GPTQ_E_INVALID_ARG;
  if (x_dtype != GPTQ_F16 && x_dtype != GPTQ_BF16) return GPTQ_E_INVALID_ARG;
  if (path == GPTQ_PATH_AUTO) path = auto_path(h, M);
  if (path != GPTQ_PATH_SKINNY && path != GPTQ_PATH_TILED) return GPTQ_E_INVALID_ARG;
  if (path == GPTQ_PATH_SKINNY && M > kSkinnyMaxM) return GPTQ_E_INVALID_ARG;
  if (M == 0) return GPTQ_OK;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return GPTQ_E_INVALID_ARG;
  const size_t xb = (size_t)M * h->K * 2, yb = (size_t)M * h->N * 2;
  if (overlaps(x, xb, y, yb)) return GPTQ_E_INVALID_ARG;
  if (bias) {
    const size_t be = h->scales_dtype == GPTQ_F32 ? 4 : 2;
    if (!aligned(bias, be) || overlaps(bias, (size_t)h->N * be, y, yb)) return GPTQ_E_INVALID_ARG;
  }
  size_t need = 0;
  st = gptq_workspace_size(h, M, x_dtype, path, &need);
  if (st != GPTQ_OK) return st;
  if (need > 0) {
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return GPTQ_E_WORKSPACE;
    if (overlaps(workspace, need, x, xb) || overlaps(workspace, need, y, yb)) return GPTQ_E_INVALID_ARG;
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev != h->device) return GPTQ_E_DEVICE;

  GemmCall c{h, x, M, x_dtype == GPTQ_BF16 ? 1 : 0, y, workspace, workspace_bytes, (hipStream_t)stream, bias};
  e = path == GPTQ_PATH_SKINNY ? launch_skinny(c) : launch_tiled(c);
  if (e != hipSuccess) return hip_fail(e);
  return GPTQ_OK;
}

gptq_status gptq_gemm(gptq_handle_t h, const void* x, int64_t M, int32_t x_dtype, void* y,
                      void* workspace, size_t workspace_bytes, int32_t path, void* stream) {
  return gemm_impl(h, x, M, x_dtype, nullptr, y, workspace, workspace_bytes, path, stream);
}

gptq_status gptq_gemm_bias(gptq_handle_t h, const void* x, int64_t M, int32_t x_dtype, const void* bias, void* y,
                           void* workspace, size_t workspace_bytes, int32_t path, void* stream) {
  return gemm_impl(h, x, M, x_dtype, bias, y, workspace, workspace_bytes, path, stream);
}

gptq_status gptq_gemm_noalloc(gptq_handle_t h, const void* x, int64_t M, int32_t x_dtype, const void* bias, void* y,
                              int32_t path, void* stream) {
  gptq_status st = check_handle(h);
  if (st != GPTQ_OK) return st;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev != h->device) return GPTQ_E_DEVICE;
  void* ws = nullptr;
  st = scratch_of_device(dev, &ws);              // one-time set-up per device (no allocation)
  if (st != GPTQ_OK) return st;
  size_t need = 0;
  st = gptq_workspace_size(h, M, x_dtype, path, &need);
  if (st != GPTQ_OK) return st;
  if (need > kScratchBytes) return GPTQ_E_SCRATCH_LIMIT;
  return gemm_impl(h, x, M, x_dtype, bias, y, ws, kScratchBytes, path, stream);
}

gptq_status gptq_destroy(gptq_handle_t h) {
  if (!h) return GPTQ_OK;
  if (!retire_handle(h)) return GPTQ_E_INVALID_ARG;   // destroyed already, or never issued
  int cur = -1;
  (void)hipGetDevice(&cur);
  if (cur != h->device) (void)hipSetDevice(h->device);
  hipError_t e = hipDeviceSynchronize();
  free_layer(h);
  if (cur >= 0 && cur != h->device) (void)hipSetDevice(cur);
  return e == hipSuccess ? GPTQ_OK : hip_fail(e);
}

gptq_status gptq_info(gptq_handle_t h, gptq_handle_info* info) {
  gptq_status st = check_handle(h);
  if (st != GPTQ_OK) return st;
  if (!info) return GPTQ_E_INVALID_ARG;
  info->in_features = h->K;
  info->out_features = h->N;
  info->bits = h->ckpt_bits;
  info->group_size = h->group_size;
  info->groups = h->G;
  info->padded_in_features = h->Kp;
  info->has_perm = h->has_perm;
  info->scales_dtype = h->scales_dtype;
  info->runtime_bytes = h->bytes;
  info->device = h->device;
  return GPTQ_OK;
}

gptq_status gptq_decode_runtime(gptq_handle_t h, uint8_t* codes_kn_host, int32_t* zeros_gn_host,
                                uint32_t* scales_gn_host, int32_t* perm_host) {
  gptq_status st = check_handle(h);
  if (st != GPTQ_OK) return st;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e);
  const int K = h->K, N = h->N, G = h->G, bits = h->bits;
  std::vector<int32_t> perm(h->Kp);
  if (h->perm) {
    e = hipMemcpy(perm.data(), h->perm, sizeof(int32_t) * h->Kp, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e);
  } else {
    for (int k = 0; k < h->Kp; ++k) perm[k] = k < K ? k : -1;
  }
  if (perm_host) std::memcpy(perm_host, perm.data(), sizeof(int32_t) * K);
  if (codes_kn_host) {
    const size_t nw = (size_t)h->CT * h->KC * unit_words(bits);
    std::vector<uint32_t> w(nw);
    e = hipMemcpy(w.data(), h->wq, nw * 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e);
    for (int ct = 0; ct < h->CT; ++ct)
      for (int kc = 0; kc < h->KC; ++kc) {
        const uint32_t* u = w.data() + ((size_t)ct * h->KC + kc) * unit_words(bits);
        for (int lane = 0; lane < kLanes; ++lane)
          for (int i = 0; i < 32; ++i) {
            Piece p[kMaxPieces];
            int np = code_pieces(bits, i, p);
            uint32_t code = 0;
            for (int q = 0; q < np; ++q) {
              uint32_t word = u[unit_word_offset(bits, lane, p[q].word)];
              code |= ((word >> p[q].bit) & ((1u << p[q].nb) - 1)) << p[q].cbit;
            }
            const int ks = kc * kChunkK + code_k_in_chunk(lane, i);
            const int n = ct * kTileN + lane_col(lane);
            if (ks < K) codes_kn_host[(size_t)perm[ks] * N + n] = (uint8_t)code;
          }
      }
  }
  const size_t meta_n = (size_t)h->CT * G * kTileN;
  if (zeros_gn_host || scales_gn_host) {
    const bool f32 = h->scales_dtype == GPTQ_F32;
    std::vector<uint32_t> meta(meta_n), s32(f32 ? meta_n : 0);
    e = hipMemcpy(meta.data(), h->meta, meta_n * 4, hipMemcpyDeviceToHost);
    if (e == hipSuccess && f32) e = hipMemcpy(s32.data(), h->scale32, meta_n * 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e);
    for (int ct = 0; ct < h->CT; ++ct)
      for (int g = 0; g < G; ++g)
        for (int j = 0; j < kTileN; ++j) {
          const size_t src = ((size_t)ct * G + g) * kTileN + j, dst = (size_t)g * N + ct * kTileN + j;
          if (zeros_gn_host) zeros_gn_host[dst] = (int32_t)(((meta[src] >> 16) + 1) & 0xFFFF);
          if (scales_gn_host) scales_gn_host[dst] = f32 ? s32[src] : (meta[src] & 0xFFFF);
        }
  }
  return GPTQ_OK;
}

gptq_status gptq_read_floor(const void* p, size_t bytes, uint32_t* sink, void* stream) {
  if (!p || !sink || bytes == 0 || bytes % 16 != 0 || !aligned(p, 16) || !aligned(sink, 4) ||
      bytes / 16 > (size_t(1) << 36))
    return GPTQ_E_INVALID_ARG;
  hipError_t e = launch_read_floor(p, bytes, sink, (hipStream_t)stream);
  return e == hipSuccess ? GPTQ_OK : hip_fail(e);
}

const char* gptq_status_str(gptq_status s) {
  switch (s) {
    case GPTQ_OK: return "ok";
    case GPTQ_E_INVALID_ARG: return "invalid argument";
    case GPTQ_E_SHAPE: return "tensor shape does not match the layer (GPTQ-002/003)";
    case GPTQ_E_GIDX: return "g_idx length or index out of range (GPTQ-004)";
    case GPTQ_E_UNSUPPORTED: return "unsupported bits, format, group size or g_idx structure";
    case GPTQ_E_HIP: return "HIP runtime error";
    case GPTQ_E_OOM: return "out of device memory";
    case GPTQ_E_WORKSPACE: return "workspace too small or misaligned";
    case GPTQ_E_NUMERIC: return "the damped Hessian is not positive definite";
    case GPTQ_E_DEVICE: return "no gfx950 device, or handle used on another device";
    case GPTQ_E_SCRATCH_LIMIT:
      return "the call needs more scratch than gptq_gemm_noalloc's static buffer holds (use gptq_gemm with a workspace)";
  }
  return "unknown status";
}

int32_t gptq_last_hip_error(void) { return t_last_hip; }

}  // extern "C"
