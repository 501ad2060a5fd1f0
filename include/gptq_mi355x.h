/*
 * gptq_mi355x.h -- C ABI of the GPTQ weight-only quantized linear layer for AMD MI355X (gfx950).
 *
 *     y[M, N] = x[M, K] . dequant(qweight, qzeros, scales, g_idx)^T
 *     W[n, k] = (code[k, n] - zero[g, n]) * scale[g, n],   g = g_idx[k]
 *
 * The operation is defined on "39. Quantized checkpoints: GPTQ, AWQ, FP8, FP4 and trellis codes",
 * section "GPTQ" / "The format" (tensor shapes, stored-minus-one zeros, the dequant equation, and
 * sorting the inputs by g_idx once at load time), and on "GPTQ packed checkpoint (safetensors /
 * torch)", sections "GptqLayer", "QuantizeConfig", "Reader" and "Reject the file when".
 * The split into a load-time repack that builds a kernel-private runtime layout and a per-call
 * GEMM follows "Kernel Backends Reference", section "Packed storage and execution concepts"
 * (runtime ABI, post_init).
 *
 * Conventions that hold for every entry point:
 *  - Every tensor pointer is a DEVICE pointer on the HIP device that is current when the call
 *    is made, unless its name ends in _host.  The caller owns every buffer it passes.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *  - Errors are returned as gptq_status, never by abort().  All argument and shape checks run
 *    before any device work, so a failed call has launched nothing and changed no output.
 *    There is no silent fallback to another kernel, dtype or layout.
 *  - A HIP runtime failure returns GPTQ_E_HIP; gptq_last_hip_error() returns its hipError_t for
 *    the calling thread.
 *  - The library is thread-safe for calls on distinct handles.  A handle is immutable after
 *    gptq_repack, so gptq_gemm may run on one handle from several streams at once as long as
 *    each call has its own workspace.  Handles are checked against the set of live handles: a
 *    destroyed or never-issued pointer returns GPTQ_E_INVALID_ARG.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gptq_layer* gptq_handle_t;

typedef enum {
  GPTQ_OK = 0,
  GPTQ_E_INVALID_ARG = 1, /* NULL / misaligned pointer, M < 0, bad dtype or path, y aliasing x */
  GPTQ_E_SHAPE = 2,       /* rule GPTQ-002 / GPTQ-003: qweight, qzeros or scales shape wrong,
                             in_features or out_features not a multiple of 32 */
  GPTQ_E_GIDX = 3,        /* rule GPTQ-004: g_idx length wrong or an index outside [0, G) */
  GPTQ_E_UNSUPPORTED = 4, /* rule GPTQ-001 (bits not 2/3/4/8, or 2..8 for GPTQ_P), GPTQ-005 (a
                             private layout such as
                             marlin), an AWQ_GEMM layer that is not 4-bit or sets desc_act,
                             group_size not -1 and not a positive multiple of 32, or a
                             g_idx whose groups are not whole (its stable sort is not j // gs) */
  GPTQ_E_HIP = 5,         /* a HIP runtime call failed (see gptq_last_hip_error) */
  GPTQ_E_OOM = 6,         /* device allocation for the runtime layout failed */
  GPTQ_E_WORKSPACE = 7,   /* workspace smaller than gptq_workspace_size() or not 256-B aligned */
  GPTQ_E_DEVICE = 8,      /* no gfx950 device, or the handle lives on another device */
  GPTQ_E_NUMERIC = 9,     /* gptq_quantize: the damped Hessian is not positive definite */
  GPTQ_E_SCRATCH_LIMIT = 10 /* gptq_gemm_noalloc: the call needs more than
                               GPTQ_NOALLOC_SCRATCH_BYTES of scratch */
} gptq_status;

/* Size of the static scratch buffer behind gptq_gemm_noalloc (bytes, per device). */
#define GPTQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

typedef enum { GPTQ_F16 = 0, GPTQ_BF16 = 1, GPTQ_F32 = 2 } gptq_dtype;

/* Checkpoint formats.  Every accepted format repacks into the same runtime layout; MARLIN (a
 * private runtime layout) is named so that callers can pass what the checkpoint declares and be
 * refused with GPTQ_E_UNSUPPORTED (rule GPTQ-005). */
typedef enum {
  GPTQ_FORMAT_GPTQ = 0,      /* AutoGPTQ "cuda" pack, 2/3/4/8-bit, v1 stored-minus-one zeros    */
  GPTQ_FORMAT_MARLIN = 1,
  /* The same words with the corrected zeros newer tools call gptq_v2 ("39. Quantized
   * checkpoints ...", section "GPTQ"; "Kernel Backends Reference", section "Packed storage and
   * execution concepts"): zero = the stored field, no "minus one".  2/3/4/8-bit. */
  GPTQ_FORMAT_GPTQ_V2 = 2,
  /* AutoAWQ GEMM tensors ("39. Quantized checkpoints: GPTQ, AWQ, FP8, FP4 and trellis codes",
   * section "AWQ"): 4-bit only; qweight int32 [K, N/8] and qzeros int32 [G, N/8] hold eight
   * fields along the OUTPUT dimension in the order 0 2 4 6 1 3 5 7 (field j of word w is output
   * 8w + order[j]); zeros are stored as they are (no "minus one"); scales [G, N]; sequential
   * groups g = k / group_size, so no g_idx.  Same W = (code - zero) * scale, same runtime layout. */
  GPTQ_FORMAT_AWQ_GEMM = 3,
  /* GPTQ_P planar words ("Kernel Backends Reference", section "Planar packing"), 2..8-bit: each
   * 32 codes take `bits` consecutive words (qweight rows, qzeros columns), one group of words per
   * plane of widths 2 | 2+1 | 4 | 4+1 | 4+2 | 4+2+1 | 8, low bits first; inside a plane the
   * fields are packed continuously, low bits first.  Zeros keep the v1 "minus one".  Shapes as
   * GPTQ.  Every width runs in a runtime layout of its own width (5/6/7-bit codes included), so
   * a call reads bits / 8 bytes per weight. */
  GPTQ_FORMAT_GPTQ_P = 4
} gptq_format;

/* Kernel family for gptq_gemm.  AUTO picks SKINNY (the streaming kernels) for M <= 8, TILED (the
 * MFMA tiles) above 32 rows, and in between whichever measured faster for the layer's shape: the
 * streaming kernel where it reads x from L2, the tiled family where its K slices are long while
 * the streaming split would cut K into many short slices.  Forcing a family is for tests; SKINNY
 * runs M <= 64 only (GPTQ_E_INVALID_ARG above), TILED any M.  Every family meets the same
 * tolerance, so the choice changes time, not results beyond rounding. */
typedef enum { GPTQ_PATH_AUTO = 0, GPTQ_PATH_SKINNY = 1, GPTQ_PATH_TILED = 2 } gptq_path;

/* Description of one checkpoint layer.  The *_shape fields are the shapes of the tensors the
 * caller holds; they are checked against K, N, bits and group_size (rules GPTQ-002..004). */
typedef struct {
  int32_t in_features;       /* K                                                              */
  int32_t out_features;      /* N                                                              */
  int32_t bits;              /* 2, 3, 4 or 8 (GPTQ-001); 2 .. 8 for GPTQ_P                     */
  int32_t group_size;        /* -1 = one group over all K, else a positive multiple of 32      */
  int32_t desc_act;          /* informational; act-order is taken from g_idx itself (must be 0
                                for AWQ_GEMM, which has no g_idx)                              */
  int32_t checkpoint_format; /* gptq_format                                                    */
  int32_t scales_dtype;      /* gptq_dtype of `scales`: F16, BF16 or F32                        */
  int32_t reserved;          /* must be 0                                                      */
  int64_t qweight_shape[2];  /* must be [K / 32 * bits, N] ([K, N / 8] for AWQ_GEMM)           */
  int64_t qzeros_shape[2];   /* must be [G, N / 32 * bits], G = ceil(K / group_size)
                                ([G, N / 8] for AWQ_GEMM)                                      */
  int64_t scales_shape[2];   /* must be [G, N]                                                 */
  int64_t g_idx_len;         /* K, or 0 when no g_idx is passed (then g = k / group_size); 0
                                for AWQ_GEMM                                                   */
} gptq_layer_desc;

typedef struct {
  int32_t in_features, out_features, bits, group_size, groups;
  int32_t padded_in_features; /* K rounded up to a multiple of 128 (the kernels' K chunk)      */
  int32_t has_perm;           /* 1 when the load-time sort of g_idx is not the identity        */
  int32_t scales_dtype;
  int64_t runtime_bytes;      /* device bytes owned by the handle                              */
  int32_t device;             /* HIP ordinal the handle lives on                               */
} gptq_handle_info;

/* Host-only check of a layer description and (optionally) a host copy of g_idx, with the same
 * rules gptq_repack applies ("GPTQ packed checkpoint", "Reject the file when").  Needs no GPU.
 * g_idx_host may be NULL (sequential groups).  Returns GPTQ_OK or the first failing status. */
gptq_status gptq_validate(const gptq_layer_desc* desc, const int32_t* g_idx_host);

/* Load-time repack (the runtime initialisation after loading).  Reads the checkpoint tensors
 *   qweight int32 [K*bits/32, N], qzeros int32 [G, N*bits/32], scales [G, N] (desc->scales_dtype),
 *   g_idx int32 [K] or NULL,
 * all device pointers, row-major, 4-byte aligned; validates them (this copies g_idx to the host
 * once); computes the stable sort of the inputs by g_idx; and builds the kernel-private runtime
 * layout in device memory owned by the new handle.  Work is queued on `stream`, which is
 * synchronised before return, so the caller may free or change the checkpoint tensors afterwards
 * (the handle does not alias them; changed tensors need a new repack).  On failure *out is NULL. */
gptq_status gptq_repack(const gptq_layer_desc* desc, const int32_t* qweight, const int32_t* qzeros,
                        const void* scales, const int32_t* g_idx, void* stream, gptq_handle_t* out);

/* Device bytes of workspace gptq_gemm needs for this handle, M, activation dtype and path
 * (0 when none).  "Kernel Backends Reference", section "Marlin and caller-owned scratch" (its
 * scratch API): the caller may supply the GEMM's scratch, the size query and the GEMM share one
 * size calculation, and supplied scratch that is too small or misaligned makes the GEMM fail
 * rather than fall back -- here gptq_gemm calls this same function and returns GPTQ_E_WORKSPACE.
 * The size depends only on (handle, M, x_dtype, path): act-order layers need a sorted copy of x;
 * the TILED family also copies x when in_features is not a multiple of 128 (rows zero-padded)
 * and, for BF16 activations, makes that copy fp16 (exactly rescaled per row by a power of two)
 * with one exponent per row; calls split along K add their fp32 partial sums.
 * Errors: GPTQ_E_INVALID_ARG (handle not live, bytes NULL, M < 0, bad dtype or path, SKINNY with
 * M > 64).  Host-only: touches no device memory. */
gptq_status gptq_workspace_size(gptq_handle_t h, int64_t M, int32_t x_dtype, int32_t path,
                                size_t* bytes);

/* y = x . W^T for the handle's layer.
 *   x  [M, K] row-major, dtype x_dtype (F16 or BF16), 16-byte aligned;
 *   y  [M, N] row-major, same dtype as x, 16-byte aligned, must not overlap x or the workspace;
 *   workspace: device memory of at least gptq_workspace_size() bytes, 256-byte aligned
 *              (may be NULL when that size is 0); its contents are scratch, and two calls in
 *              flight at once must not share one workspace.
 * Accumulates in fp32 and rounds y to x_dtype with round-to-nearest-even.  M == 0 returns
 * GPTQ_OK with nothing launched ("Formats and kernels ...", the zero-token forward of an idle
 * data-parallel rank).  Queues work on `stream` only: no allocation, no synchronisation, so the
 * call can be captured in a HIP graph. */
gptq_status gptq_gemm(gptq_handle_t h, const void* x, int64_t M, int32_t x_dtype, void* y,
                      void* workspace, size_t workspace_bytes, int32_t path, void* stream);

/* y = x . W^T + bias: gptq_gemm with the layer's optional bias vector added ("GPTQ packed
 * checkpoint (safetensors / torch)", section "GptqLayer": an [out_features] tensor in the same
 * dtype as the scales, applied at the layer's output).
 *   bias  [N] device vector in the handle's scales dtype (F16 or BF16: 2-byte aligned; F32:
 *         4-byte aligned), read only, must not overlap y; NULL makes the call identical to
 *         gptq_gemm.
 * The bias is added in fp32 to each output's accumulated sum, before the one rounding to x_dtype.
 * Everything else (arguments, workspace, errors, graph capture) is as for gptq_gemm. */
gptq_status gptq_gemm_bias(gptq_handle_t h, const void* x, int64_t M, int32_t x_dtype, const void* bias, void* y,
                           void* workspace, size_t workspace_bytes, int32_t path, void* stream);

/* gptq_gemm_bias (bias may be NULL, then it is gptq_gemm) for callers that cannot allocate or pass
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The call's scratch (the sorted or fp16 copy of x, row exponents, split-K partial
 * sums) lives in a static device buffer of GPTQ_NOALLOC_SCRATCH_BYTES (32 MiB) that the library
 * holds on every device it runs on until the process ends; no device memory is allocated or freed
 * by this call, and no workspace is passed.  The first call on a device (a call with M == 0 will do)
 * looks up that device's buffer once; later calls only launch kernels.
 * Every call on one device shares that device's buffer and leaves its last contents there (nothing
 * in it needs to start at zero): calls that may overlap in time on one device -- on different
 * streams, or from different threads -- race on it and must be ordered by the caller (one stream,
 * or events).  gptq_gemm with its own workspace has no such restriction.
 * Arguments, layouts, results and other errors are those of gptq_gemm_bias.  Errors:
 * GPTQ_E_SCRATCH_LIMIT when gptq_workspace_size() for this (handle, M, x_dtype, path) exceeds the
 * buffer (nothing is launched; typically prefill-sized M: use gptq_gemm with a workspace), and
 * GPTQ_E_DEVICE when the current device is not the handle's. */
gptq_status gptq_gemm_noalloc(gptq_handle_t h, const void* x, int64_t M, int32_t x_dtype, const void* bias, void* y,
                              int32_t path, void* stream);

/* Frees the handle's device memory after synchronising its device.  "Kernel Backends Reference",
 * "Kernel implementation and validation checklist" item 5: a runtime handle must be invalidated
 * when the layer it was built from changes -- a changed checkpoint needs gptq_destroy and a new
 * gptq_repack (the handle never aliases the checkpoint tensors).  The library keeps the set of
 * live handles: after this call the pointer is no longer live, and any later call with it
 * (gptq_destroy included) returns GPTQ_E_INVALID_ARG without reading the freed memory.  NULL is
 * accepted (GPTQ_OK).  Errors: GPTQ_E_INVALID_ARG (not a live handle), GPTQ_E_HIP (the device
 * synchronisation failed; the memory is freed regardless). */
gptq_status gptq_destroy(gptq_handle_t h);

/* Handle properties.  "Kernel Backends Reference", section "Packed storage and execution concepts":
 * after the runtime initialisation a layer no longer exposes the checkpoint's tensors, so this is
 * where callers read what the runtime layout holds -- the layer's sizes, groups, padded input
 * width, whether a load-time permutation is in effect, and runtime_bytes, the device memory the
 * handle owns (the section "Pitfalls" warns against estimating memory from checkpoint bytes).
 * Errors: GPTQ_E_INVALID_ARG (handle not live, info NULL).  Host-only. */
gptq_status gptq_info(gptq_handle_t h, gptq_handle_info* info);

/* Test hook: reads the runtime layout back and decodes it on the host into the checkpoint's
 * logical values, in ORIGINAL input order.  "Kernel Backends Reference", "Kernel implementation and
 * validation checklist" item 6 asks repack changes to be checked against an independent oracle;
 * this is how tests compare the runtime layout with the oracle's unpack, bit for bit.  The section
 * "Pitfalls" says a private runtime layout must not be saved under a checkpoint format: this hook
 * returns logical values, never the runtime words.
 *   codes_kn_host  uint8 [K * N]  code[k, n] at k * N + n
 *   zeros_gn_host  int32 [G * N]  zero[g, n] (GPTQ: stored + 1; AWQ_GEMM: as stored)
 *   scales_gn_host uint32 [G * N] raw scale bits (16-bit patterns zero-extended, or f32 bits)
 *   perm_host      int32 [K]      input index at each sorted position
 * Any output pointer may be NULL to skip it.  Synchronises the device.  The runtime layout is
 * not a checkpoint and must not be saved as one. */
gptq_status gptq_decode_runtime(gptq_handle_t h, uint8_t* codes_kn_host, int32_t* zeros_gn_host,
                                uint32_t* scales_gn_host, int32_t* perm_host);

/* Device read floor: reads `bytes` of device memory at p once and discards them (sink, 4 bytes of
 * device memory, is written only for a value the data cannot produce).  "Formats and kernels: FP8,
 * INT8, INT4, Marlin, Machete", opening section, prices a small-M call of a weight-only layer by the
 * time to stream its packed weight bytes; this is that stream alone, for timing a layer's call
 * against the device's own read rate at the same byte count.  p 16-byte aligned, bytes a positive
 * multiple of 16 (at most 2^40), queued on `stream`, no synchronisation.
 * Errors: GPTQ_E_INVALID_ARG, GPTQ_E_HIP. */
gptq_status gptq_read_floor(const void* p, size_t bytes, uint32_t* sink, void* stream);

/* Static message for a status code, naming the rule of "GPTQ packed checkpoint (safetensors /
 * torch)", section "Reject the file when", where a status stands for one (GPTQ-001 .. GPTQ-005).
 * Unknown codes give "unknown status".  Never NULL; the string is owned by the library. */
const char* gptq_status_str(gptq_status s);

/* hipError_t behind the calling thread's last GPTQ_E_HIP (0 if none).  Thread-local: a failure is
 * reported to the thread that made the call, never silently replaced by another path ("Kernel
 * Backends Reference", section "Marlin and caller-owned scratch": failures are reported, not
 * papered over by a fallback). */
int32_t gptq_last_hip_error(void);

/* ---- GPTQ quantizer: the step that produces a layer's codes -------------------------------------
 * "39. Quantized checkpoints: GPTQ, AWQ, FP8, FP4 and trellis codes", section "GPTQ".  All tensor
 * pointers are DEVICE pointers on the current device, row-major; calls are stream-ordered. */

/* H[K, K] (float32) = 2 X^T X / S for calibration inputs x [S, K] (x_dtype F16, BF16 or F32): the
 * Hessian every output row shares.  Sums in float64, rounded once.  H is overwritten; K <= 32768.
 * Errors: GPTQ_E_INVALID_ARG (NULL, S or K out of range, bad dtype), GPTQ_E_HIP. */
gptq_status gptq_hessian(const void* x, int64_t S, int32_t K, int32_t x_dtype, float* H, void* stream);

typedef struct {
  int32_t bits;        /* 2 .. 8: codes in [0, 2^bits - 1]                                      */
  int32_t group_size;  /* -1 (one group) or a positive multiple of 32, counted in visiting order */
  int32_t act_order;   /* 1: visit inputs from the largest H_ii down (desc_act)                  */
  float damp;          /* fraction of the mean diagonal added to H's diagonal (the page: 0.01)  */
  int32_t reserved;    /* must be 0                                                             */
} gptq_quant_params;

/* Device workspace gptq_quantize needs for an [N, K] layer (256-byte aligned). */
gptq_status gptq_quantize_workspace_size(int32_t N, int32_t K, size_t* bytes);

/* Quantize W [N, K] (float32, rows are outputs) against H [K, K] (float32, e.g. from gptq_hessian)
 * with the page's GPTQ: never-active inputs (H_ii = 0) zeroed, optional act-order, damped Cholesky
 * inverse, per-column error feedback through the upper Cholesky factor of H^-1 in blocks of 128
 * columns with one update product per block, group grids from the corrected weights.  Grid of a
 * group (a reading; the page names the step only): asymmetric min-max over each row's group values
 * widened to contain 0: scale = (hi - lo) / (2^bits - 1), zero = round(-lo / scale).
 * Outputs (device, caller-owned): codes uint8 [N, K] in the ORIGINAL input order, scales float32
 * [N, G] and zeros int32 [N, G] (the logical zero, 0 .. 2^bits - 1; a zero of 0 needs
 * GPTQ_FORMAT_GPTQ_V2 to be stored) with G = ceil(K / group_size), g_idx int32 [K] (group of each
 * input).  W and H are read only.  Synchronises the stream.  Uses rocSOLVER (POTRF, TRTRI) and
 * rocBLAS (SGEMM), loaded on first use.
 * Errors: GPTQ_E_INVALID_ARG (NULL, reserved != 0, damp outside [0, 1]), GPTQ_E_UNSUPPORTED (bits,
 * group_size, or the solver libraries not found), GPTQ_E_SHAPE (K not a multiple of 32 or > 16384,
 * N > 2^20, N * K > 2^31), GPTQ_E_WORKSPACE, GPTQ_E_NUMERIC, GPTQ_E_HIP. */
gptq_status gptq_quantize(const float* W, const float* H, int32_t N, int32_t K, const gptq_quant_params* params,
                          uint8_t* codes, float* scales, int32_t* zeros, int32_t* g_idx, void* workspace,
                          size_t workspace_bytes, void* stream);

/* The checkpoint writer ("39. Quantized checkpoints ...", section "GPTQ": codes along the input
 * dimension low bits first, zeros along the output dimension, scales [groups, out]): logical codes
 * uint8 [N, K], scales float32 [N, G] and zeros int32 [N, G] (as gptq_quantize returns them) ->
 * qweight int32 [K / 32 * bits, N], qzeros int32 [G, N / 32 * bits] and scales_out [G, N] in
 * scales_dtype (F16 / BF16 rounded to nearest even, or F32), for checkpoint_format GPTQ (v1: the
 * stored zero is (zero - 1) & mask, so a zero of 0 reads back as 2^bits, the format's own quirk),
 * GPTQ_V2 (zeros as they are) or GPTQ_P (planar words, v1 zeros; 2..8-bit).  Device pointers,
 * stream-ordered, no synchronisation.  Errors: GPTQ_E_INVALID_ARG, GPTQ_E_UNSUPPORTED (format,
 * bits, group_size), GPTQ_E_SHAPE (N or K not a multiple of 32, or out of range), GPTQ_E_HIP. */
gptq_status gptq_pack(const uint8_t* codes, const float* scales, const int32_t* zeros, int32_t N, int32_t K,
                      int32_t bits, int32_t group_size, int32_t checkpoint_format, int32_t scales_dtype,
                      int32_t* qweight, int32_t* qzeros, void* scales_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GPTQ_MI355X_H */
