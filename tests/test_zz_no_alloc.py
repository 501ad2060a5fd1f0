"""gptq_gemm_noalloc (the entry point for callers that cannot allocate: static per-device scratch)
against gptq_gemm with a caller workspace, through the C ABI: the same kernels on the same inputs,
so the outputs must be bitwise equal -- on two calls in a row, the second with a smaller input (the
buffer keeps the first call's contents), on calls whose scratch holds a sorted / fp16 copy of x
and split-K partial sums.  A call that needs more than the buffer is refused without a launch."""
import ctypes
import sys

import numpy as np
import pytest

import gptq_inputs as gi
from gpu_util import bits_to_device, device_to_bits, repack_layer, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_only_quantized_amd as wq
    wq.load_library()
    yield


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def call_ref(lib, h, x, M, xcode, y, ws, path, s, bias=None):
    if bias is None:
        return lib.gptq_gemm(h.ptr, x.data_ptr(), M, xcode, y.data_ptr(), ws.data_ptr(), ws.numel(), path, s)
    return lib.gptq_gemm_bias(h.ptr, x.data_ptr(), M, xcode, bias.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(),
                              path, s)


def call_noalloc(lib, h, x, M, xcode, y, path, s, bias=None):
    return lib.gptq_gemm_noalloc(h.ptr, x.data_ptr(), M, xcode, None if bias is None else bias.data_ptr(),
                                 y.data_ptr(), path, s)


# (label, K, N, bits, gs, desc_act, x dtype, path, (M first, M second), bias)
CASES = [
    ("mid split K", 8192, 2048, 4, 128, False, "bf16", 1, (16, 9), False),
    ("tiled bf16 prep + split K", 4096, 2048, 4, 128, False, "bf16", 2, (64, 40), False),
    ("act-order prep + tiled", 2048, 1024, 3, 64, True, "f16", 0, (96, 33), False),
    ("act-order mid", 4096, 1024, 2, 128, True, "bf16", 1, (24, 5), True),
    ("skinny staged (no scratch)", 4096, 2048, 4, 128, False, "f16", 0, (1, 1), False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_workspace_call(case):
    import torch
    import weight_only_quantized_amd as wq
    lib = wq.load_library()
    label, K, N, bits, gs, act, xdt, path, Ms, with_bias = case
    say("noalloc", label, Ms)
    L = gi.make_layer(K, N, bits, gs, desc_act=act, scales_dtype="f16", seed=gi.seed_for(8, bits))
    h = repack_layer(L)
    tdt = torch_dtype(xdt)
    xcode = wq.F16 if xdt == "f16" else wq.BF16
    s = torch.cuda.current_stream().cuda_stream
    bias = bits_to_device(gi.make_bias(N, "f16", seed=gi.seed_for(8, 3)), "f16") if with_bias else None
    for i, M in enumerate(Ms):
        x = bits_to_device(gi.make_x(M, K, xdt, seed=gi.seed_for(8, 10 + i)), xdt)
        need = h.workspace_size(M, tdt, path)
        assert need <= wq.NOALLOC_SCRATCH_BYTES
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        y_ref = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
        y = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
        assert call_ref(lib, h, x, M, xcode, y_ref, ws, path, s, bias) == 0
        st = call_noalloc(lib, h, x, M, xcode, y, path, s, bias)
        assert st == 0, wq.STATUS.get(st)
        torch.cuda.synchronize()
        assert np.array_equal(device_to_bits(y), device_to_bits(y_ref)), (label, M)
    h.close()


def test_noalloc_refuses_calls_beyond_its_buffer_and_m0():
    import torch
    import weight_only_quantized_amd as wq
    lib = wq.load_library()
    K, N, M = 8192, 1024, 4096            # a bf16 prefill: the fp16 copy of x alone is 64 MiB
    L = gi.make_layer(K, N, 4, 128, desc_act=False, scales_dtype="f16", seed=gi.seed_for(8, 20))
    h = repack_layer(L)
    assert h.workspace_size(M, torch.bfloat16, wq.PATH_TILED) > wq.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    st = lib.gptq_gemm_noalloc(h.ptr, x.data_ptr(), M, wq.BF16, None, y.data_ptr(), wq.PATH_TILED, s)
    assert wq.STATUS[st] == "E_SCRATCH_LIMIT"
    assert b"static buffer" in lib.gptq_status_str(st)
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))                      # nothing was launched
    assert lib.gptq_gemm_noalloc(h.ptr, x.data_ptr(), 0, wq.BF16, None, y.data_ptr(), 0, s) == 0   # M = 0
    h.close()
    assert wq.STATUS[lib.gptq_gemm_noalloc(h._ptr or ctypes.c_void_p(1), x.data_ptr(), 1, wq.BF16, None,
                                           y.data_ptr(), 0, s)] == "E_INVALID_ARG"
