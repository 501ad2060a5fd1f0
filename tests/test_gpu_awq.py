"""GPU parity of the AutoAWQ GEMM repack source: the same runtime layout and kernels, fed by the
4-bit AWQ pack (fields along the output dimension, zeros as stored).

Repack must be bit-exact against the oracle's AWQ unpack; GEMM output is held to the same bar as
the GPTQ layers (rel-L2 <= 1e-3 fp16 / 4e-3 bf16, max-abs <= 2e-2 * rms) against gemm_awq."""
import sys

import numpy as np
import pytest

import oracle as o
import gptq_inputs as gi
from gpu_util import bits_to_device, check, repack_awq_layer, run_gemm

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


@pytest.mark.parametrize("K,N,gs,sdt", [(256, 256, 128, "f16"), (4096, 128, 128, "bf16"),
                                        (288, 96, 32, "f32"), (512, 64, -1, "f16"), (96, 32, 32, "bf16")])
def test_awq_repack_decodes_to_oracle_unpack(K, N, gs, sdt):
    say("awq-repack", K, N, gs, sdt)
    L = gi.make_awq_layer(K, N, gs, sdt, seed=K + 3 * N)
    h = repack_awq_layer(L)
    d = h.decode()
    assert np.array_equal(d["codes"], o.unpack_awq(L.qweight))
    assert np.array_equal(d["zeros"], o.unpack_awq(L.qzeros).astype(np.int32))
    want_sc = L.scales.view(np.uint32) if sdt == "f32" else L.scales.astype(np.uint32)
    assert np.array_equal(d["scales"], want_sc)
    assert np.array_equal(d["perm"], np.arange(K))
    assert h.info()["has_perm"] == 0
    h.close()


MS = [1, 2, 3, 5, 16, 17, 33, 64, 65, 130]


@pytest.mark.parametrize("K,N,gs,sdt,xdt", [(160, 96, 32, "f16", "f16"), (384, 288, 128, "bf16", "bf16"),
                                            (544, 64, -1, "f32", "f16"), (256, 160, 64, "f16", "bf16")])
def test_awq_gemm_small_shapes_both_paths(K, N, gs, sdt, xdt):
    import weight_only_quantized_amd as wq
    say("awq-gemm-small", K, N, gs, sdt, xdt)
    L = gi.make_awq_layer(K, N, gs, sdt, seed=5 * K + N)
    h = repack_awq_layer(L)
    x = gi.make_x(max(MS), K, xdt, seed=K + N)
    y_ref = o.gemm_awq(x, xdt, L.qweight, L.qzeros, L.scales, sdt, gs)
    for M in MS:
        for p in [wq.PATH_TILED] + ([wq.PATH_SKINNY] if M <= 64 else []):
            check(run_gemm(h, x[:M], xdt, path=p), xdt, y_ref[:M], label=(M, p))
    h.close()


DISPATCH_MS = [1, 2, 4, 5, 16, 33, 64, 130, 257]


@pytest.mark.parametrize("K,xdt", [(4096, "f16"), (4096, "bf16"), (8192, "f16"), (8192, "bf16")])
def test_awq_gemm_dispatch_variants(K, xdt):
    """Long K selects the straight-line skinny variants (with the bf16 offset form at M = 1), the
    split-K mid kernel and the tiled kernel, as for GPTQ layers."""
    import weight_only_quantized_amd as wq
    N = 96
    say("awq-dispatch", K, xdt)
    L = gi.make_awq_layer(K, N, 128, "f16", seed=K + 1)
    h = repack_awq_layer(L)
    x = gi.make_x(max(DISPATCH_MS), K, xdt, seed=K + 2)
    y_ref = o.gemm_awq(x, xdt, L.qweight, L.qzeros, L.scales, "f16", 128)
    for M in DISPATCH_MS:
        for p in [wq.PATH_AUTO] + ([wq.PATH_SKINNY] if M <= 64 else []):
            check(run_gemm(h, x[:M], xdt, path=p), xdt, y_ref[:M], label=(K, xdt, M, p))
    h.close()


@pytest.mark.parametrize("zero", [0, 15])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_awq_extreme_zeros(zero, xdt):
    """Every zero 0 (only AWQ stores it: the runtime record holds 0xFFFF) or every zero 15, with
    random codes, on every family."""
    import weight_only_quantized_amd as wq
    K, N, gs = 2048, 128, 128
    say("awq-zero", zero, xdt)
    base = gi.make_awq_layer(K, N, gs, "f16", seed=99 + zero)
    qz = o.pack_awq(np.full((K // gs, N), zero))
    L = gi.AwqLayer(K, N, gs, base.qweight, qz, base.scales, "f16")
    h = repack_awq_layer(L)
    assert np.all(h.decode()["zeros"] == zero)
    x = gi.make_x(130, K, xdt, seed=7)
    y_ref = o.gemm_awq(x, xdt, L.qweight, L.qzeros, L.scales, "f16", gs)
    for M in (1, 4, 33, 130):
        for p in [wq.PATH_AUTO, wq.PATH_TILED] + ([wq.PATH_SKINNY] if M <= 64 else []):
            check(run_gemm(h, x[:M], xdt, path=p), xdt, y_ref[:M], label=(zero, M, p))
    h.close()


def test_awq_bias():
    import weight_only_quantized_amd as wq
    K, N = 1024, 256
    L = gi.make_awq_layer(K, N, 128, "bf16", seed=4)
    h = repack_awq_layer(L)
    b = gi.make_bias(N, "bf16", seed=5)
    x = gi.make_x(40, K, "bf16", seed=6)
    y_ref = o.gemm_awq(x, "bf16", L.qweight, L.qzeros, L.scales, "bf16", 128) + o.decode_float_bits(b, "bf16")
    for M in (1, 9, 40):
        for p in (wq.PATH_AUTO, wq.PATH_TILED):
            check(run_gemm(h, x[:M], "bf16", path=p, bias=b, bias_tag="bf16"), "bf16", y_ref[:M], label=(M, p))
    h.close()


def test_awq_rejects_what_the_format_cannot_hold():
    import torch
    import weight_only_quantized_amd as wq
    L = gi.make_awq_layer(256, 64, 64, "f16", seed=3)
    qw = torch.from_numpy(L.qweight).cuda()
    qz = torch.from_numpy(L.qzeros).cuda()
    sc = bits_to_device(L.scales, "f16")
    g = torch.from_numpy((np.arange(256) // 64).astype(np.int32)).cuda()
    cases = [
        (dict(bits=4, group_size=64, checkpoint_format="awq_gemm", desc_act=True), None, "E_UNSUPPORTED"),
        (dict(bits=8, group_size=64, checkpoint_format="awq_gemm"), None, "E_UNSUPPORTED"),
        (dict(bits=4, group_size=64, checkpoint_format="awq_gemm"), g, "E_GIDX"),
    ]
    for kw, gidx, name in cases:
        with pytest.raises(wq.GPTQError) as e:
            wq.repack(qw, qz, sc, gidx, **kw)
        assert e.value.name == name, (kw, e.value.name)
    with pytest.raises(wq.GPTQError) as e:      # qzeros of the wrong width
        wq.repack(qw, qz[:, :2].contiguous(), sc, None, bits=4, group_size=64, checkpoint_format="awq_gemm")
    assert e.value.name == "E_SHAPE"
