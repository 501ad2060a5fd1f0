"""Python binding of the GPTQ weight-only quantized linear layer for MI355X (gfx950).

The binding only marshals arguments: it passes device pointers of torch tensors and the current
HIP stream to the C ABI declared in include/gptq_mi355x.h.  Every step of the layer runs in the
library's HIP kernels.  If the library is not built, importing still works but every call raises.
There is no CPU or PyTorch fallback.

    h = repack(qweight, qzeros, scales, g_idx, bits=4, group_size=128)
    y = h.gemm(x)          # x [M, K] fp16/bf16 on the GPU -> y [M, N], same dtype
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["LIB_PATH", "GPTQError", "Desc", "Handle", "load_library", "repack", "validate", "symbols",
           "STATUS", "PATH_AUTO", "PATH_SKINNY", "PATH_TILED"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgptq_mi355x.so")

STATUS = {0: "OK", 1: "E_INVALID_ARG", 2: "E_SHAPE", 3: "E_GIDX", 4: "E_UNSUPPORTED", 5: "E_HIP",
          6: "E_OOM", 7: "E_WORKSPACE", 8: "E_DEVICE", 9: "E_NUMERIC", 10: "E_SCRATCH_LIMIT"}
NOALLOC_SCRATCH_BYTES = 32 << 20    # GPTQ_NOALLOC_SCRATCH_BYTES
F16, BF16, F32 = 0, 1, 2
FORMATS = {"gptq": 0, "marlin": 1, "gptq_v2": 2, "awq_gemm": 3, "gptq_p": 4}
PATH_AUTO, PATH_SKINNY, PATH_TILED = 0, 1, 2

# Every symbol include/gptq_mi355x.h declares.
symbols = ["gptq_validate", "gptq_repack", "gptq_workspace_size", "gptq_gemm", "gptq_gemm_bias", "gptq_gemm_noalloc",
           "gptq_destroy",
           "gptq_info", "gptq_decode_runtime", "gptq_status_str", "gptq_last_hip_error", "gptq_hessian",
           "gptq_quantize_workspace_size", "gptq_quantize", "gptq_pack", "gptq_read_floor"]


class GPTQError(RuntimeError):
    def __init__(self, status, where, lib=None):
        msg = STATUS.get(status, str(status))
        if lib is not None:
            msg += ": " + lib.gptq_status_str(status).decode()
            if status == 5:
                msg += f" (hipError {lib.gptq_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class QuantParams(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("act_order", ctypes.c_int32),
                ("damp", ctypes.c_float), ("reserved", ctypes.c_int32)]


class Desc(ctypes.Structure):
    _fields_ = [("in_features", ctypes.c_int32), ("out_features", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("desc_act", ctypes.c_int32), ("checkpoint_format", ctypes.c_int32),
                ("scales_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("qweight_shape", ctypes.c_int64 * 2), ("qzeros_shape", ctypes.c_int64 * 2),
                ("scales_shape", ctypes.c_int64 * 2), ("g_idx_len", ctypes.c_int64)]


class Info(ctypes.Structure):
    _fields_ = [("in_features", ctypes.c_int32), ("out_features", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("groups", ctypes.c_int32), ("padded_in_features", ctypes.c_int32),
                ("has_perm", ctypes.c_int32), ("scales_dtype", ctypes.c_int32), ("runtime_bytes", ctypes.c_int64),
                ("device", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the built library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                           "or `python weight_only_quantized_amd/build.py`")
    # torch first: the library then binds to the HIP runtime torch has loaded, so both share one
    # runtime (a library loaded before torch would bring up a second runtime in the process)
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.gptq_validate.argtypes = [ctypes.POINTER(Desc), P]
    lib.gptq_repack.argtypes = [ctypes.POINTER(Desc), P, P, P, P, P, ctypes.POINTER(P)]
    lib.gptq_workspace_size.argtypes = [P, I64, I32, I32, ctypes.POINTER(SZ)]
    lib.gptq_gemm.argtypes = [P, P, I64, I32, P, P, SZ, I32, P]
    lib.gptq_gemm_bias.argtypes = [P, P, I64, I32, P, P, P, SZ, I32, P]
    lib.gptq_gemm_noalloc.argtypes = [P, P, I64, I32, P, P, I32, P]
    lib.gptq_destroy.argtypes = [P]
    lib.gptq_info.argtypes = [P, ctypes.POINTER(Info)]
    lib.gptq_decode_runtime.argtypes = [P, P, P, P, P]
    lib.gptq_status_str.argtypes = [I32]
    lib.gptq_status_str.restype = ctypes.c_char_p
    lib.gptq_last_hip_error.argtypes = []
    lib.gptq_hessian.argtypes = [P, I64, I32, I32, P, P]
    lib.gptq_quantize_workspace_size.argtypes = [I32, I32, ctypes.POINTER(SZ)]
    lib.gptq_quantize.argtypes = [P, P, I32, I32, ctypes.POINTER(QuantParams), P, P, P, P, P, SZ, P]
    lib.gptq_pack.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, P]
    lib.gptq_read_floor.argtypes = [P, SZ, P, P]
    for f in ("gptq_validate", "gptq_repack", "gptq_workspace_size", "gptq_gemm", "gptq_gemm_bias", "gptq_gemm_noalloc",
              "gptq_destroy",
              "gptq_info", "gptq_decode_runtime", "gptq_last_hip_error", "gptq_hessian",
              "gptq_quantize_workspace_size", "gptq_quantize", "gptq_pack", "gptq_read_floor"):
        getattr(lib, f).restype = I32
    _lib = lib
    return lib


def _dtype_code(dt) -> int:
    import torch
    if dt == torch.float16:
        return F16
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {dt}")


def make_desc(K, N, bits, group_size, scales_dtype, qweight_shape, qzeros_shape, scales_shape, g_idx_len,
              desc_act=False, checkpoint_format="gptq") -> Desc:
    d = Desc()
    d.in_features, d.out_features, d.bits, d.group_size = K, N, bits, group_size
    d.desc_act = int(bool(desc_act))
    d.checkpoint_format = FORMATS[checkpoint_format] if isinstance(checkpoint_format, str) else int(checkpoint_format)
    d.scales_dtype = scales_dtype
    d.reserved = 0
    d.qweight_shape[:] = list(qweight_shape)
    d.qzeros_shape[:] = list(qzeros_shape)
    d.scales_shape[:] = list(scales_shape)
    d.g_idx_len = g_idx_len
    return d


def validate(desc: Desc, g_idx_host=None) -> int:
    """Host-only validation (needs no GPU).  g_idx_host: a numpy int32 array or None.  Returns the status."""
    lib = load_library()
    ptr = None
    if g_idx_host is not None:
        import numpy as np
        g = np.ascontiguousarray(g_idx_host, dtype=np.int32)
        ptr = g.ctypes.data_as(ctypes.c_void_p)
        return lib.gptq_validate(ctypes.byref(desc), ptr)
    return lib.gptq_validate(ctypes.byref(desc), None)


class _OnStream:
    """Run one library call on `stream` (default: the current stream).  When that is not the
    current stream, it first waits for the current stream (which produced the inputs), tensors
    created inside the block are allocated on it, and `keep(t)` records caller tensors on it so
    that torch's caching allocator does not hand their memory to other work while the call may
    still read or write them."""

    def __init__(self, stream, device):
        import torch
        self.cur = torch.cuda.current_stream(device)
        self.stream = stream if stream is not None else self.cur
        self.side = self.stream.cuda_stream != self.cur.cuda_stream
        self._ctx = torch.cuda.stream(self.stream)

    def __enter__(self):
        if self.side:
            self.stream.wait_stream(self.cur)
        self._ctx.__enter__()
        return self

    def __exit__(self, *exc):
        return self._ctx.__exit__(*exc)

    def keep(self, *tensors):
        if self.side:
            for t in tensors:
                if t is not None:
                    t.record_stream(self.stream)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.stream.cuda_stream)


class Handle:
    """A repacked layer living on one GPU.  Owns the runtime layout until close()."""

    def __init__(self, lib, ptr, K, N, bits, group_size):
        self._lib, self._ptr = lib, ptr
        self.K, self.N, self.bits, self.group_size = K, N, bits, group_size

    @property
    def ptr(self):
        if not self._ptr:
            raise RuntimeError("handle is closed")
        return self._ptr

    def info(self) -> dict:
        inf = Info()
        st = self._lib.gptq_info(self.ptr, ctypes.byref(inf))
        if st:
            raise GPTQError(st, "gptq_info", self._lib)
        return {f: getattr(inf, f) for f, _ in Info._fields_}

    def workspace_size(self, M, dtype, path=PATH_AUTO) -> int:
        n = ctypes.c_size_t(0)
        st = self._lib.gptq_workspace_size(self.ptr, M, _dtype_code(dtype), path, ctypes.byref(n))
        if st:
            raise GPTQError(st, "gptq_workspace_size", self._lib)
        return n.value

    def gemm(self, x, out=None, workspace=None, path=PATH_AUTO, stream=None, bias=None):
        """y = x . W^T (+ bias); x [M, K] fp16/bf16 on this handle's GPU; bias, when given, an [N]
        tensor in the scales' dtype (gptq_gemm_bias).  `workspace` (uint8 tensor) is allocated from
        torch's caching allocator when not given.  With `stream` (a torch stream) the call runs on
        it after the current stream's pending work; two calls in flight at once need workspaces of
        their own."""
        import torch
        if x.dim() != 2 or x.shape[1] != self.K:
            raise ValueError(f"x must be [M, {self.K}]")
        if out is not None and (tuple(out.shape) != (x.shape[0], self.N) or out.dtype != x.dtype
                                or not out.is_contiguous()):
            raise ValueError("out must be a contiguous [M, N] tensor of x's dtype")
        if bias is not None:
            if bias.dim() != 1 or bias.shape[0] != self.N or not bias.is_contiguous():
                raise ValueError(f"bias must be a contiguous [{self.N}] tensor")
            if _dtype_code(bias.dtype) != self.info()["scales_dtype"]:
                raise TypeError("bias must have the scales' dtype")
        M = x.shape[0]
        need = self.workspace_size(M, x.dtype, path)
        with _OnStream(stream, x.device) as on:
            on.keep(x, out, workspace, bias)
            x = x.contiguous()
            if out is None:
                out = torch.empty((M, self.N), dtype=x.dtype, device=x.device)
            if workspace is None and need:
                workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
            ws_ptr = workspace.data_ptr() if workspace is not None else None
            ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
            if bias is None:
                st = self._lib.gptq_gemm(self.ptr, x.data_ptr(), M, _dtype_code(x.dtype), out.data_ptr(), ws_ptr,
                                         ws_n, path, on.ptr)
                where = "gptq_gemm"
            else:
                st = self._lib.gptq_gemm_bias(self.ptr, x.data_ptr(), M, _dtype_code(x.dtype), bias.data_ptr(),
                                              out.data_ptr(), ws_ptr, ws_n, path, on.ptr)
                where = "gptq_gemm_bias"
        if st:
            raise GPTQError(st, where, self._lib)
        return out

    def decode(self) -> dict:
        """Test hook: the runtime layout decoded back to logical codes / zeros / scale bits / perm."""
        import numpy as np
        codes = np.zeros((self.K, self.N), dtype=np.uint8)
        inf = self.info()
        G = inf["groups"]
        zeros = np.zeros((G, self.N), dtype=np.int32)
        scales = np.zeros((G, self.N), dtype=np.uint32)
        perm = np.zeros(self.K, dtype=np.int32)
        st = self._lib.gptq_decode_runtime(self.ptr, codes.ctypes.data, zeros.ctypes.data, scales.ctypes.data,
                                           perm.ctypes.data)
        if st:
            raise GPTQError(st, "gptq_decode_runtime", self._lib)
        return {"codes": codes, "zeros": zeros, "scales": scales, "perm": perm}

    def close(self):
        if self._ptr:
            st = self._lib.gptq_destroy(self._ptr)
            self._ptr = None
            if st:
                raise GPTQError(st, "gptq_destroy", self._lib)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def repack(qweight, qzeros, scales, g_idx=None, *, bits, group_size, desc_act=False, checkpoint_format="gptq",
           stream=None) -> Handle:
    """Build the runtime layout from checkpoint tensors on the current GPU (int32 qweight/qzeros,
    fp16/bf16/fp32 scales, optional int32 g_idx).  The inputs may be freed afterwards.
    checkpoint_format "awq_gemm" reads AutoAWQ GEMM tensors instead (4-bit, qweight [K, N/8],
    qzeros [G, N/8], zeros as stored, no g_idx), "gptq_v2" GPTQ words with zeros as stored, and
    "gptq_p" GPTQ_P planar words (2..8-bit, v1 zeros)."""
    import torch
    lib = load_library()
    for name, t in (("qweight", qweight), ("qzeros", qzeros), ("scales", scales)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if qweight.dtype != torch.int32 or qzeros.dtype != torch.int32:
        raise TypeError("qweight and qzeros must be int32")
    awq = FORMATS.get(checkpoint_format, checkpoint_format) == FORMATS["awq_gemm"]
    if awq:  # AutoAWQ GEMM: qweight [K, N / 8], eight 4-bit fields per word along the outputs
        K, N = qweight.shape[0], qweight.shape[1] * 8
    else:
        K = qweight.shape[0] * 32 // bits if 2 <= bits <= 8 else 0
        N = qweight.shape[1]
    if g_idx is not None:
        if g_idx.dtype != torch.int32 or not g_idx.is_cuda or not g_idx.is_contiguous():
            raise TypeError("g_idx must be a contiguous int32 GPU tensor")
        K = g_idx.shape[0]
    d = make_desc(K, N, bits, group_size, _dtype_code(scales.dtype), qweight.shape, qzeros.shape, scales.shape,
                  0 if g_idx is None else g_idx.shape[0], desc_act, checkpoint_format)
    out = ctypes.c_void_p()
    with _OnStream(stream, qweight.device) as on:       # gptq_repack synchronises its stream
        st = lib.gptq_repack(ctypes.byref(d), qweight.data_ptr(), qzeros.data_ptr(), scales.data_ptr(),
                             None if g_idx is None else g_idx.data_ptr(), on.ptr, ctypes.byref(out))
    if st:
        raise GPTQError(st, "gptq_repack", lib)
    return Handle(lib, out, K, N, bits, group_size)


def hessian(x, stream=None):
    """H = 2 X^T X / S (float32 [K, K]) of calibration inputs x [S, K] (fp16/bf16/fp32 GPU tensor)."""
    import torch
    lib = load_library()
    if not x.is_cuda or not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous 2-D GPU tensor")
    S, K = x.shape
    with _OnStream(stream, x.device) as on:
        on.keep(x)
        H = torch.empty((K, K), dtype=torch.float32, device=x.device)
        st = lib.gptq_hessian(x.data_ptr(), S, K, _dtype_code(x.dtype), H.data_ptr(), on.ptr)
    if st:
        raise GPTQError(st, "gptq_hessian", lib)
    return H


def quantize(W, H, *, bits=4, group_size=128, act_order=False, damp=0.01, stream=None):
    """GPTQ-quantize W [N, K] (float32 GPU tensor) against H [K, K] on the GPU.  Returns (codes uint8
    [N, K], scales float32 [N, G], zeros int32 [N, G], g_idx int32 [K]) as torch GPU tensors."""
    import torch
    lib = load_library()
    for name, t in (("W", W), ("H", H)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    N, K = W.shape
    if tuple(H.shape) != (K, K):
        raise ValueError("H must be [K, K]")
    G = 1 if group_size == -1 else -(-K // group_size)
    dev = W.device
    n = ctypes.c_size_t(0)
    st = lib.gptq_quantize_workspace_size(N, K, ctypes.byref(n))
    if st:
        raise GPTQError(st, "gptq_quantize_workspace_size", lib)
    p = QuantParams(bits, group_size, int(bool(act_order)), float(damp), 0)
    with _OnStream(stream, dev) as on:                  # gptq_quantize synchronises its stream
        codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
        scales = torch.empty((N, G), dtype=torch.float32, device=dev)
        zeros = torch.empty((N, G), dtype=torch.int32, device=dev)
        g_idx = torch.empty((K,), dtype=torch.int32, device=dev)
        ws = torch.empty(n.value, dtype=torch.uint8, device=dev)
        st = lib.gptq_quantize(W.data_ptr(), H.data_ptr(), N, K, ctypes.byref(p), codes.data_ptr(),
                               scales.data_ptr(), zeros.data_ptr(), g_idx.data_ptr(), ws.data_ptr(), n.value, on.ptr)
    if st:
        raise GPTQError(st, "gptq_quantize", lib)
    return codes, scales, zeros, g_idx


def pack(codes, scales, zeros, *, bits, group_size, checkpoint_format="gptq_v2", scales_dtype=None, stream=None):
    """Write quantizer outputs (codes uint8 [N, K], scales float32 [N, G], zeros int32 [N, G], GPU
    tensors) as checkpoint tensors on the GPU: (qweight int32 [K*bits/32, N], qzeros int32
    [G, N*bits/32], scales [G, N] in scales_dtype, default float16)."""
    import torch
    lib = load_library()
    N, K = codes.shape
    G = scales.shape[1]
    sdt = torch.float16 if scales_dtype is None else scales_dtype
    dev = codes.device
    fmt = FORMATS[checkpoint_format] if isinstance(checkpoint_format, str) else int(checkpoint_format)
    with _OnStream(stream, dev) as on:
        on.keep(codes, scales, zeros)
        qweight = torch.empty((K * bits // 32, N), dtype=torch.int32, device=dev)
        qzeros = torch.empty((G, N * bits // 32), dtype=torch.int32, device=dev)
        s_out = torch.empty((G, N), dtype=sdt, device=dev)
        st = lib.gptq_pack(codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), N, K, bits, group_size, fmt,
                           _dtype_code(sdt), qweight.data_ptr(), qzeros.data_ptr(), s_out.data_ptr(), on.ptr)
    if st:
        raise GPTQError(st, "gptq_pack", lib)
    return qweight, qzeros, s_out
