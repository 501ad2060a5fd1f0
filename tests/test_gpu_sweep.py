"""GPU parity on a seeded sweep of layer shapes around the dispatcher's boundaries: every row count
from 1 to 33 and a few beyond 64, on layers long enough for the workgroup's copy of x to come in
parts, with every code width, group size, scale dtype and activation dtype, with and without
act-order.  Each case runs the automatic kernel choice and the two forced families against the
float64 oracle, to the same bars as the other parity tests."""
import sys

import numpy as np
import pytest

import oracle as o
import gptq_inputs as gi
from gpu_util import check, repack_layer, run_gemm

pytestmark = pytest.mark.gpu

_ROWS = [1, 2, 3, 4, 5, 7, 8, 9, 12, 15, 16, 17, 20, 24, 31, 32, 33, 48, 64, 65, 100]


def _cases():
    rng = np.random.default_rng(20261203)
    cases = []
    for i in range(80):
        K = int(rng.choice([1024, 1056, 2048, 3072, 4064, 4096, 5120, 6144, 8192]))
        N = int(rng.choice([256, 512, 768, 1024, 1536, 2048]))
        while K * N > 4 * 1024 * 1024:          # keeps the oracle's float64 product in seconds
            N //= 2
        bits = int(rng.choice([2, 3, 4, 8]))
        gs = int(rng.choice([32, 64, 128, 128, 256, -1]))
        desc = bool(rng.integers(0, 3) == 0)
        sdt = str(rng.choice(["f16", "bf16", "f32"]))
        xdt = str(rng.choice(["f16", "bf16"]))
        Ms = sorted(set(int(m) for m in rng.choice(_ROWS, size=5, replace=False)))
        cases.append((i, K, N, bits, gs, desc, sdt, xdt, tuple(Ms)))
    return cases


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("i,K,N,bits,gs,desc,sdt,xdt,Ms", _cases())
def test_sweep(i, K, N, bits, gs, desc, sdt, xdt, Ms):
    import weight_only_quantized_amd as wq
    print("sweep", i, K, N, bits, gs, desc, sdt, xdt, Ms, flush=True)
    L = gi.make_layer(K, N, bits, gs, desc_act=desc, scales_dtype=sdt, seed=1000 + i)
    h = repack_layer(L)
    x = gi.make_x(max(Ms), K, xdt, seed=2000 + i)
    y_ref = o.gemm(x, xdt, L.qweight, L.qzeros, L.scales, sdt, L.g_idx, bits)
    for M in Ms:
        paths = [wq.PATH_AUTO, wq.PATH_TILED] + ([wq.PATH_SKINNY] if M <= 64 else [])
        for p in paths:
            y = run_gemm(h, x[:M], xdt, path=p)
            check(y, xdt, y_ref[:M], label=(i, K, N, bits, gs, desc, sdt, xdt, M, p))
    h.close()
