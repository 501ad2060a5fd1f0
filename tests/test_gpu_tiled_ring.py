"""GPU parity of the tiled kernel's two-chunks-in-flight forms, call after call.

Each wave of these forms loads its share of the next chunks' x tile into registers and writes it to
LDS itself, and the workgroup publishes it with a barrier after a counted wait.  With the pieces
loaded by LDS DMA under the same counted wait, the 64-row tile in eight waves read 16 stale rows of
x in about half of its calls (on MI355X), so every form is run several times here, each result
against the float64 oracle: the 16-row tile, the 32-row tile (eight waves), the 64-row tile in
four waves and in eight (small grids, and every grid with 8-bit codes), with and without act-order.
"""
import numpy as np
import pytest

import oracle as o
import gptq_inputs as gi
from gpu_util import check, repack_layer, run_gemm

pytestmark = pytest.mark.gpu

REPS = 6

# (K, N, M, bits, group size, act-order, x dtype): the tile each one takes is in its comment
CASES = [
    (4096, 4096, 16, 4, 128, False, "f16"),     # 16 x 128
    (8192, 1024, 32, 4, 128, False, "bf16"),    # 32 x 128, eight waves
    (8192, 2048, 32, 2, 128, True, "f16"),      # 32 x 128 after the sorted copy of x
    (8192, 4096, 64, 4, 128, False, "f16"),     # 64 x 128, four waves (over 256 workgroups)
    (8192, 128, 64, 4, 128, False, "f16"),      # 64 x 128, eight waves (small grid)
    (2048, 4096, 128, 4, 128, False, "bf16"),   # short K, 64 x 128 in eight waves
    (8192, 8192, 48, 8, 128, False, "f16"),     # 64 x 128 over 256 workgroups, 8-bit: eight waves
    (4096, 8192, 40, 3, 64, True, "f16"),       # 64 x 128, four waves, after the sorted copy of x
    (4096, 2048, 40, 3, 64, True, "bf16"),      # 64 x 128, eight waves, after the sorted copy of x
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("K,N,M,bits,gs,desc,xdt", CASES)
def test_two_chunk_ring_every_call(K, N, M, bits, gs, desc, xdt):
    import weight_only_quantized_amd as wq
    print("tiled-ring", K, N, M, bits, gs, desc, xdt, flush=True)
    L = gi.make_layer(K, N, bits, gs, desc_act=desc, scales_dtype="f16", seed=K + N + M + bits)
    h = repack_layer(L)
    x = gi.make_x(M, K, xdt, seed=K + M + 1)
    y_ref = o.gemm(x, xdt, L.qweight, L.qzeros, L.scales, "f16", L.g_idx, bits)
    for rep in range(REPS):
        y = run_gemm(h, x, xdt, path=wq.PATH_TILED)
        check(y, xdt, y_ref, label=(K, N, M, bits, gs, desc, xdt, rep))
    h.close()


@pytest.mark.parametrize("K", [128, 256, 512, 640, 1152])
def test_two_chunk_tiles_every_tail(K):
    """Slices of 1, 2, 4, 5 and 9 chunks (K unsplit): no full step of three, the two tail steps
    alone, one step of three and one or two tail steps, three steps of three and no tail.  The
    36864-column layer gives the 64-row tile more than 256 workgroups (its four-wave form), and 16
    rows take the 16-row tile."""
    import weight_only_quantized_amd as wq
    print("tiled-tail", K, flush=True)
    N = 36864
    L = gi.make_layer(K, N, 4, 128, scales_dtype="f16", seed=K + 7)
    h = repack_layer(L)
    for xdt in ("f16", "bf16"):
        x = gi.make_x(64, K, xdt, seed=K + 8)
        y_ref = o.gemm(x, xdt, L.qweight, L.qzeros, L.scales, "f16", L.g_idx, 4)
        for M in (16, 64):
            y = run_gemm(h, x[:M], xdt, path=wq.PATH_TILED)
            check(y, xdt, y_ref[:M], label=(K, xdt, M))
    h.close()
