"""Plain float64 CPU oracle for y = x . dequant(qweight, qzeros, scales, g_idx)^T.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy, float64, no
blocking or fusion beyond what the definitions below state.

Sources (page title, then section):
  [FMT]  "39. Quantized checkpoints: GPTQ, AWQ, FP8, FP4 and trellis codes",
         section "GPTQ", sub-part "The format" (tensor shapes, "stored minus one"
         zeros, the dequant equation, sorting inputs by g_idx at load time) and
         its pack / unpack / as_int32 helpers (the writer and the two's-complement
         wrap).
  [SPEC] "GPTQ packed checkpoint (safetensors / torch)", sections "GptqLayer"
         (shapes, ceil(in/group) groups, the optional [out_features] bias in the
         scales' dtype), "QuantizeConfig" (bits 2/3/4/8,
         group_size -1 = one group), "Reader" (low bits first along the input
         dimension, the "10 / split / 10" 3-bit loop, +1 on unpacked zeros,
         W = (code - zero) * scale with g = g_idx[k]) and "Reject the file when"
         (rules GPTQ-001 .. GPTQ-006).
  [KBR]  "Kernel Backends Reference" (GPTQModel wiki), section "Packed storage and
         execution concepts" (group size -1, desc_act / g_idx, v1 zero semantics)
         and "Kernel implementation and validation checklist" (separate arithmetic
         error from output-rounding error).
  [FK]   "Formats and kernels: FP8, INT8, INT4, Marlin, Machete", opening section
         (effective bits b_eff = bits + 16 / group_size with fp16 scales).
  [PLN]  "Kernel Backends Reference", section "Planar packing": GPTQ_P words -- a b-bit
         code (b = 2 .. 8) split into planes of widths 2 | 2+1 | 4 | 4+1 | 4+2 | 4+2+1 | 8,
         low bits first; each plane width divides 32 so no field straddles a word; the
         plane words of every 32 codes are adjacent, low plane first; single-plane 2/4/8
         are bit-identical to continuous packing, planar 3-bit is not.
  [V2]   "39. Quantized checkpoints ...", section "GPTQ" (the corrected layout newer tools
         call gptq_v2: no "minus one" on stored zeros) and "Kernel Backends Reference",
         section "Packed storage and execution concepts" (v1 / v2 zero semantics).
  [AWQ]  "39. Quantized checkpoints: GPTQ, AWQ, FP8, FP4 and trellis codes", section
         "AWQ", its checkpoint part: AutoAWQ GEMM tensors qweight [in, out / 8] and
         qzeros [groups, out / 8] pack eight 4-bit fields along the OUTPUT dimension in
         the interleaved order 0 2 4 6 1 3 5 7 (output 1's field in bits 16-19), zeros
         are stored as they are (offset = -zero * scale), scales [groups, out].

Readings where the pages are silent or ambiguous:
  * v1 zeros: the writer stores (z - 1) & mask, the reader adds 1 with no mask,
    so a stored all-ones field reads back as 2**bits ([FMT] writer vs reader;
    [SPEC] GPTQ-006).
  * 3-bit: each 32 codes form one little-endian 96-bit stream over three
    consecutive words (code j at stream bits 3j .. 3j+2); code 10 straddles words
    0/1 and code 21 straddles words 1/2 -- the "10 / split / 10" of [SPEC].  The
    same stream rule packs qzeros along the output dimension.
  * int32 words are two's-complement images of 32-bit fields ([FMT] as_int32);
    fields are read with logical shifts of the unsigned image.
  * group_size = -1 means one group covering all inputs ([SPEC] QuantizeConfig).
  * GPTQ_P: inside a plane, code j of a block of 32 sits at bit w*j mod 32 of the plane's
    word w*j // 32 (continuous packing of that plane, which is what makes single-plane
    layouts identical to continuous ones); the same rule packs qzeros along the output
    dimension; its zeros keep the GPTQ (v1) "minus one" ([PLN] names only the packing).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "SUPPORTED_BITS", "num_groups", "to_u32", "to_i32",
    "unpack_along_rows", "unpack_along_cols", "pack_along_rows", "pack_along_cols",
    "unpack_codes", "unpack_zeros", "pack_codes", "pack_zeros",
    "decode_float_bits", "round_to_dtype_bits", "validate_layer",
    "dequant", "gemm", "gemm_bias", "gemm_entries", "runtime_perm", "compare", "effective_bits",
    "AWQ_ORDER", "unpack_awq", "pack_awq", "dequant_awq", "gemm_awq",
    "PLANES", "planar_unpack_rows", "planar_pack_rows", "planar_unpack_cols", "planar_pack_cols",
    "FORMATS", "dequant_fmt", "gemm_fmt",
]

SUPPORTED_BITS = (2, 3, 4, 8)          # [SPEC] QuantizeConfig / GPTQ-001


def num_groups(K: int, group_size: int) -> int:
    """G = ceil(in_features / group_size); group_size = -1 is one group ([SPEC] GptqLayer,
    QuantizeConfig)."""
    if group_size == -1:
        return 1
    return -(-K // group_size)


def to_u32(words) -> np.ndarray:
    """Unsigned 32-bit image of int32 words, held in int64 ([FMT] as_int32 is its inverse)."""
    return np.asarray(words).astype(np.int64) & 0xFFFFFFFF


def to_i32(u) -> np.ndarray:
    """32 bits held in an int64 -> int32 with the same bits (two's complement), [FMT] as_int32."""
    u = np.asarray(u, dtype=np.int64)
    return (((u + 2 ** 31) % 2 ** 32) - 2 ** 31).astype(np.int32)


# ----------------------------------------------------------------------------------------------
# Bit fields.  A "row-packed" array holds codes along axis 0 ([SPEC] Reader: pack = 32 // bits
# codes per qweight row, low bits first); a "column-packed" one holds them along axis 1 (qzeros).
# ----------------------------------------------------------------------------------------------

def _field_from_stream(w: np.ndarray, bit: int, bits: int) -> np.ndarray:
    """Read the `bits`-wide field that starts at stream bit `bit` of a little-endian stream of
    32-bit words w[0], w[1], ... (w indexed along axis 0)."""
    wi, sh = divmod(bit, 32)
    mask = (1 << bits) - 1
    v = w[wi] >> sh
    if sh + bits > 32:                       # the field straddles into the next word
        v = v | (w[wi + 1] << (32 - sh))
    return v & mask


def unpack_along_rows(words, bits: int) -> np.ndarray:
    """int32 [R, C] -> codes [R * 32 // bits, C] (int64).

    bits in {2, 4, 8}: row r holds codes r*pack .. r*pack+pack-1, code j at bits
    bits*j .. bits*j+bits-1 ([SPEC] Reader; [FMT] "low bits first").
    bits == 3: rows 3t, 3t+1, 3t+2 form one 96-bit stream holding codes 32t .. 32t+31,
    code j at stream bits 3j .. 3j+2 (the "10 / split / 10" reading).
    """
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"unsupported bits {bits}")
    u = to_u32(words)
    R, C = u.shape
    if bits == 3:
        if R % 3:
            raise ValueError("3-bit packing needs a multiple of 3 rows")
        out = np.empty((R // 3 * 32, C), dtype=np.int64)
        for t in range(R // 3):
            w = u[3 * t: 3 * t + 3]
            for j in range(32):
                out[32 * t + j] = _field_from_stream(w, 3 * j, 3)
        return out
    pack = 32 // bits
    out = np.empty((R * pack, C), dtype=np.int64)
    for j in range(pack):
        out[j::pack] = (u >> (bits * j)) & ((1 << bits) - 1)
    return out


def unpack_along_cols(words, bits: int) -> np.ndarray:
    """int32 [R, C] -> codes [R, C * 32 // bits]: the same stream rule along axis 1."""
    return unpack_along_rows(np.asarray(words).T, bits).T


def pack_along_rows(codes, bits: int) -> np.ndarray:
    """codes [K, C] (each in [0, 2**bits)) -> int32 [K * bits // 32, C]: the writer.

    Accumulates in int64 and wraps to int32 at the end, as the [FMT] writer does.
    """
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"unsupported bits {bits}")
    q = np.asarray(codes, dtype=np.int64)
    if q.min(initial=0) < 0 or q.max(initial=0) >= (1 << bits):
        raise ValueError("code out of range")
    K, C = q.shape
    if K % (32 if bits == 3 else 32 // bits):
        raise ValueError("codes do not fill whole words")
    out = np.zeros((K * bits // 32, C), dtype=np.int64)
    for j in range(K):
        # code j sits at bit (j % 32) * bits of the `bits`-word block that holds codes
        # 32*(j//32) .. 32*(j//32)+31
        base = (j // 32) * bits
        wi, sh = divmod((j % 32) * bits, 32)
        out[base + wi] |= (q[j] << sh) & 0xFFFFFFFF
        if sh + bits > 32:                    # the high part of a straddling 3-bit code
            out[base + wi + 1] |= q[j] >> (32 - sh)
    return to_i32(out)


def pack_along_cols(codes, bits: int) -> np.ndarray:
    return pack_along_rows(np.asarray(codes).T, bits).T.copy()


def unpack_codes(qweight, bits: int) -> np.ndarray:
    """qweight int32 [K*bits/32, N] -> code[k, n] ([SPEC] Reader; [FMT] unpack)."""
    return unpack_along_rows(qweight, bits)


def unpack_zeros(qzeros, bits: int) -> np.ndarray:
    """qzeros int32 [G, N*bits/32] -> zero[g, n] = stored + 1, NOT masked ([SPEC] GPTQ-006,
    Reader: `unpack_zeros(...) + 1`; [FMT] unpack "+ 1  # stored minus 1")."""
    return unpack_along_cols(qzeros, bits) + 1


def pack_codes(codes, bits: int) -> np.ndarray:
    """code[k, n] -> qweight, the [FMT] writer generalised to 2/3/4/8 bits."""
    return pack_along_rows(codes, bits)


def pack_zeros(zeros, bits: int) -> np.ndarray:
    """zero[g, n] -> qzeros with the v1 "stored minus one": (z - 1) & mask ([FMT] pack_gptq)."""
    z = (np.asarray(zeros, dtype=np.int64) - 1) & ((1 << bits) - 1)
    return pack_along_cols(z, bits)


# ----------------------------------------------------------------------------------------------
# Floating-point formats (inputs arrive as raw 16-bit patterns, or float32)
# ----------------------------------------------------------------------------------------------

def decode_float_bits(a, dtype: str) -> np.ndarray:
    """Raw fp16 / bf16 bit patterns (uint16) or float32 values -> float64 (exact)."""
    a = np.asarray(a)
    if dtype == "f16":
        return a.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_to_dtype_bits(y, dtype: str) -> np.ndarray:
    """float64 -> fp16 / bf16 bit patterns with round-to-nearest-even, done in one step from
    float64 (no double rounding).  Overflow goes to +-inf, NaN stays NaN."""
    y = np.asarray(y, dtype=np.float64)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return y.astype(np.float16).view(np.uint16)
    if dtype != "bf16":
        raise ValueError(dtype)
    out = np.empty(y.shape, dtype=np.uint16)
    flat, o = y.reshape(-1), out.reshape(-1)
    fin = np.isfinite(flat)
    v = flat[fin]
    _, e = np.frexp(v)                          # v = m * 2**e with 0.5 <= |m| < 1
    e = np.maximum(e, -125)                     # below 2**-126 the spacing is the subnormal 2**-133
    r = np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)   # 8 significant bits, RNE (np.rint is RNE)
    with np.errstate(over="ignore"):
        bits32 = r.astype(np.float32).view(np.uint32)   # exact: r has <= 8 significant bits
    big = np.abs(r) >= 2.0 ** 128
    bits32 = np.where(big, np.where(r > 0, np.uint32(0x7F800000), np.uint32(0xFF800000)), bits32)
    o[fin] = (bits32 >> 16).astype(np.uint16)
    nf = ~fin
    o[nf] = (flat[nf].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    o[np.isnan(flat)] = 0x7FC0
    return out


# ----------------------------------------------------------------------------------------------
# Validation: [SPEC] "Reject the file when" GPTQ-001..006, plus the readings in this module's docstring
# ----------------------------------------------------------------------------------------------

def validate_layer(K, N, bits, group_size, qweight_shape, qzeros_shape, scales_shape, g_idx=None,
                   checkpoint_format="gptq", desc_act=False) -> str:
    """Return "ok", "unsupported", "shape" or "gidx" for a checkpoint layer.  Formats: "gptq"
    and "gptq_v2" (2/3/4/8-bit, [SPEC] shapes), "gptq_p" (2..8-bit, the same shapes: `bits` words
    per 32 codes, [PLN]), "awq_gemm" (4-bit, qweight [K, N/8], qzeros [G, N/8], no g_idx and no
    act-order, [AWQ]); anything else (a private layout such as marlin) is GPTQ-005."""
    fmt = checkpoint_format
    if fmt not in ("gptq", "gptq_v2", "gptq_p", "awq_gemm"):            # GPTQ-005
        return "unsupported"
    allowed = tuple(range(2, 9)) if fmt == "gptq_p" else ((4,) if fmt == "awq_gemm" else SUPPORTED_BITS)
    if bits not in allowed or (fmt == "awq_gemm" and desc_act):         # GPTQ-001
        return "unsupported"
    if group_size != -1 and (group_size <= 0 or group_size % 32):       # reading: gs multiple of 32
        return "unsupported"
    if K <= 0 or K % 32 or N <= 0 or N % 32:                            # GPTQ-002
        return "shape"
    G = num_groups(K, group_size)
    if fmt == "awq_gemm":
        if tuple(qweight_shape) != (K, N // 8) or tuple(qzeros_shape) != (G, N // 8):
            return "shape"
        if g_idx is not None:
            return "gidx"
    elif tuple(qweight_shape) != (K // 32 * bits, N) or tuple(qzeros_shape) != (G, N // 32 * bits):
        return "shape"                                                  # GPTQ-002 / GPTQ-003
    if tuple(scales_shape) != (G, N):                                   # [SPEC] GptqLayer scales
        return "shape"
    if g_idx is not None:
        g = np.asarray(g_idx)
        if g.shape != (K,) or g.min() < 0 or g.max() >= G:             # GPTQ-004
            return "gidx"
        # reading: groups must be whole after the load-time sort -- the sorted g_idx must be the
        # sequential map j // group_size (what act-order GPTQ writes); anything else is refused.
        gs = K if group_size == -1 else group_size
        if not np.array_equal(np.sort(g, kind="stable"), np.arange(K) // gs):
            return "unsupported"
    return "ok"


# ----------------------------------------------------------------------------------------------
# The method
# ----------------------------------------------------------------------------------------------

def dequant(qweight, qzeros, scales, scales_dtype: str, g_idx, bits: int) -> np.ndarray:
    """W[n, k] = (code[k, n] - zero[g, n]) * scale[g, n] with g = g_idx[k], in float64
    ([FMT] the W[o, i] equation; [SPEC] Reader dequant loop).  Exact: an integer of
    magnitude <= 2**bits times a value with <= 24 significant bits."""
    code = unpack_codes(qweight, bits).astype(np.float64)      # [K, N]
    zero = unpack_zeros(qzeros, bits).astype(np.float64)       # [G, N]
    s = decode_float_bits(scales, scales_dtype)                # [G, N]
    g = np.asarray(g_idx, dtype=np.int64)
    return ((code - zero[g]) * s[g]).T.copy()                  # [N, K]


def gemm(x_bits, x_dtype: str, qweight, qzeros, scales, scales_dtype: str, g_idx, bits: int,
         chunk: int = 4096) -> np.ndarray:
    """y_ref[m, n] = sum_k x[m, k] * W[n, k] in float64 (a library float64 matmul per chunk of
    output columns; chunking only bounds memory)."""
    x = decode_float_bits(x_bits, x_dtype)                     # [M, K]
    qweight = np.asarray(qweight)
    N = qweight.shape[1]
    pack_n = 32 // bits if bits != 3 else None
    y = np.empty((x.shape[0], N), dtype=np.float64)
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        # qzeros packs along N: unpack all zeros once per chunk, then slice the columns
        zero_cols = slice(n0, n1)
        W = _dequant_cols(qweight[:, n0:n1], qzeros, scales, scales_dtype, g_idx, bits, zero_cols)
        y[:, n0:n1] = x @ W.T
    return y


def gemm_bias(x_bits, x_dtype: str, qweight, qzeros, scales, scales_dtype: str, g_idx, bits: int,
              bias_bits) -> np.ndarray:
    """y_ref[m, n] = sum_k x[m, k] * W[n, k] + bias[n] in float64: the layer with its optional
    bias ([SPEC] GptqLayer: an [out_features] tensor in the same dtype as the scales)."""
    b = decode_float_bits(bias_bits, scales_dtype)             # [N]
    return gemm(x_bits, x_dtype, qweight, qzeros, scales, scales_dtype, g_idx, bits) + b[None, :]


def _dequant_cols(qweight_cols, qzeros, scales, scales_dtype, g_idx, bits, cols):
    code = unpack_codes(qweight_cols, bits).astype(np.float64)
    zero = unpack_zeros(qzeros, bits)[:, cols].astype(np.float64)
    s = decode_float_bits(np.asarray(scales)[:, cols], scales_dtype)
    g = np.asarray(g_idx, dtype=np.int64)
    return ((code - zero[g]) * s[g]).T


def gemm_entries(x_bits, x_dtype, qweight, qzeros, scales, scales_dtype, g_idx, bits, rows, cols):
    """y_ref at the listed (rows[i], cols[i]) pairs only: the same definition, one output at a
    time, for checking samples of outputs too large to compute whole."""
    x = decode_float_bits(np.asarray(x_bits)[np.unique(rows)], x_dtype)
    row_pos = {r: i for i, r in enumerate(np.unique(rows))}
    ucols = np.unique(cols)
    W = {}
    for n in ucols:
        W[n] = _dequant_cols(np.asarray(qweight)[:, n:n + 1], qzeros, scales, scales_dtype,
                             g_idx, bits, slice(n, n + 1))[0]
    return np.array([x[row_pos[r]] @ W[c] for r, c in zip(rows, cols)], dtype=np.float64)


# ----------------------------------------------------------------------------------------------
# AWQ GEMM checkpoints: the same W = (code - zero) * scale from another packing
# ----------------------------------------------------------------------------------------------

AWQ_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)   # [AWQ] field j of a word holds output 8 w + AWQ_ORDER[j]


def _awq_shifts() -> np.ndarray:
    """Bit offset of output column c % 8 inside its word: 4 * (position of c % 8 in AWQ_ORDER)."""
    pos = np.empty(8, dtype=np.uint32)
    pos[list(AWQ_ORDER)] = np.arange(8, dtype=np.uint32)
    return 4 * pos


def unpack_awq(words) -> np.ndarray:
    """int32 [rows, cols / 8] -> uint8 codes [rows, cols]: column c is the 4-bit field at bit
    4 * pos(c % 8) of word c // 8 ([AWQ])."""
    u = to_u32(words)
    cols = u.shape[1] * 8
    sh = np.tile(_awq_shifts(), u.shape[1])                   # [cols]
    return ((u[:, np.arange(cols) // 8] >> sh[None, :]) & 0xF).astype(np.uint8)


def pack_awq(codes) -> np.ndarray:
    """Inverse of unpack_awq (used by the generators and pins only)."""
    c = np.asarray(codes, dtype=np.uint32)
    rows, cols = c.shape
    assert cols % 8 == 0 and c.max(initial=0) < 16
    sh = np.tile(_awq_shifts(), cols // 8)
    words = np.zeros((rows, cols // 8), dtype=np.uint32)
    for c8 in range(8):                                        # one field position at a time
        words |= c[:, c8::8] << sh[c8]
    return to_i32(words)


def dequant_awq(qweight, qzeros, scales, scales_dtype: str, group_size: int) -> np.ndarray:
    """W[n, k] = (code[k, n] - zero[g, n]) * scale[g, n], g = k // group_size, zeros used as
    stored ([AWQ]: offset = -zero * scale), in float64 (exact)."""
    code = unpack_awq(qweight).astype(np.float64)              # [K, N]
    zero = unpack_awq(qzeros).astype(np.float64)               # [G, N]
    s = decode_float_bits(scales, scales_dtype)                # [G, N]
    K = code.shape[0]
    g = np.arange(K) // (K if group_size == -1 else group_size)
    return ((code - zero[g]) * s[g]).T.copy()                  # [N, K]


def gemm_awq(x_bits, x_dtype: str, qweight, qzeros, scales, scales_dtype: str, group_size: int) -> np.ndarray:
    """y_ref = x . W^T for an AWQ GEMM layer, float64."""
    x = decode_float_bits(x_bits, x_dtype)
    return x @ dequant_awq(qweight, qzeros, scales, scales_dtype, group_size).T


def runtime_perm(g_idx) -> np.ndarray:
    """The load-time input order: a stable ascending sort of the inputs by g_idx, so that every
    group is contiguous ([FMT] "sorts the input columns by g_idx once at load time")."""
    return np.argsort(np.asarray(g_idx), kind="stable").astype(np.int64)


def effective_bits(K, N, bits, group_size, scale_bytes=2, with_zeros=False) -> float:
    """Stored bits per weight: 8 * bytes / (K * N) over qweight + scales (+ qzeros)."""
    G = num_groups(K, group_size)
    b = K * bits // 32 * N * 4 + G * N * scale_bytes
    if with_zeros:
        b += G * (N * bits // 32) * 4
    return 8.0 * b / (K * N)


def compare(y_bits, out_dtype: str, y_ref) -> dict:
    """Error metrics of a device result against the float64 reference ([KBR] checklist:
    arithmetic error is reported against y_ref, output-rounding error against RNE(y_ref))."""
    y = decode_float_bits(y_bits, out_dtype)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    y_rne = decode_float_bits(round_to_dtype_bits(y_ref, out_dtype), out_dtype)
    nref = np.linalg.norm(y_ref)
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    d = y - y_ref
    return {
        "rel_l2": float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d)),
        "max_abs": float(np.max(np.abs(d))) if d.size else 0.0,
        "rms_ref": rms,
        "max_abs_over_rms": float(np.max(np.abs(d)) / rms) if rms > 0 else float("inf"),
        "rel_l2_vs_rne": float(np.linalg.norm(y - y_rne) / nref) if nref > 0 else 0.0,
        "max_abs_vs_rne": float(np.max(np.abs(y - y_rne))) if d.size else 0.0,
        "nonfinite": int(np.count_nonzero(~np.isfinite(y))),
    }


# ----------------------------------------------------------------------------------------------
# GPTQ_P planar packing and GPTQ v2 zeros: the same W equation from other encodings
# ----------------------------------------------------------------------------------------------

PLANES = {2: (2,), 3: (2, 1), 4: (4,), 5: (4, 1), 6: (4, 2), 7: (4, 2, 1), 8: (8,)}   # [PLN]


def planar_unpack_rows(words, bits: int) -> np.ndarray:
    """int32 [K * bits / 32, C] -> codes [K, C] (int64) ([PLN]): rows bits*t .. bits*t + bits - 1
    hold codes 32t .. 32t + 31, plane by plane (PLANES[bits], low bits first); a plane of width w
    takes w of those rows, code j's field at bit w*(j % (32/w)) of its row j // (32/w)."""
    u = to_u32(words)
    R, C = u.shape
    if bits not in PLANES or R % bits:
        raise ValueError("planar rows must hold whole 32-code blocks")
    out = np.zeros((R // bits * 32, C), dtype=np.int64)
    for t in range(R // bits):
        row, low = bits * t, 0
        for w in PLANES[bits]:
            per = 32 // w
            for j in range(32):
                field = (u[row + j // per] >> (w * (j % per))) & ((1 << w) - 1)
                out[32 * t + j] |= field.astype(np.int64) << low
            row += w
            low += w
    return out


def planar_pack_rows(codes, bits: int) -> np.ndarray:
    """Inverse of planar_unpack_rows (used by the pins and generators of fixtures only)."""
    q = np.asarray(codes, dtype=np.int64)
    K, C = q.shape
    if bits not in PLANES or K % 32 or q.min(initial=0) < 0 or q.max(initial=0) >= (1 << bits):
        raise ValueError("codes must fill whole 32-code blocks and fit the width")
    out = np.zeros((K * bits // 32, C), dtype=np.int64)
    for t in range(K // 32):
        row, low = bits * t, 0
        for w in PLANES[bits]:
            per = 32 // w
            for j in range(32):
                field = (q[32 * t + j] >> low) & ((1 << w) - 1)
                out[row + j // per] |= field << (w * (j % per))
            row += w
            low += w
    return to_i32(out)


def planar_unpack_cols(words, bits: int) -> np.ndarray:
    return planar_unpack_rows(np.asarray(words).T, bits).T


def planar_pack_cols(codes, bits: int) -> np.ndarray:
    return planar_pack_rows(np.asarray(codes).T, bits).T.copy()


FORMATS = ("gptq", "gptq_v2", "gptq_p")


def dequant_fmt(fmt: str, qweight, qzeros, scales, scales_dtype: str, g_idx, bits: int) -> np.ndarray:
    """W[n, k] = (code[k, n] - zero[g, n]) * scale[g, n], g = g_idx[k], in float64, with codes and
    zeros read as the checkpoint format stores them:
      gptq     continuous words, zero = stored + 1 (v1)            -- dequant()
      gptq_v2  continuous words, zero = stored ([V2])
      gptq_p   planar words ([PLN]), zero = stored + 1 (v1 reading)."""
    if fmt == "gptq":
        return dequant(qweight, qzeros, scales, scales_dtype, g_idx, bits)
    if fmt == "gptq_v2":
        code, zero = unpack_codes(qweight, bits), unpack_along_cols(qzeros, bits)
    elif fmt == "gptq_p":
        code, zero = planar_unpack_rows(qweight, bits), planar_unpack_cols(qzeros, bits) + 1
    else:
        raise ValueError(fmt)
    s = decode_float_bits(scales, scales_dtype)
    g = np.asarray(g_idx, dtype=np.int64)
    return ((code.astype(np.float64) - zero.astype(np.float64)[g]) * s[g]).T.copy()


def gemm_fmt(fmt: str, x_bits, x_dtype: str, qweight, qzeros, scales, scales_dtype: str, g_idx,
             bits: int) -> np.ndarray:
    """y_ref = x . W^T for a layer of checkpoint format `fmt`, float64."""
    x = decode_float_bits(x_bits, x_dtype)
    return x @ dequant_fmt(fmt, qweight, qzeros, scales, scales_dtype, g_idx, bits).T
