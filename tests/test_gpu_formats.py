"""GPU parity of the GPTQ v2 and GPTQ_P planar repack sources: the same runtime layout and kernels
fed by other encodings of the same W (zeros stored without the "minus one"; planar words, with
5/6/7-bit codes widened to the 8-bit runtime layout).

Repack must be bit-exact against the oracle's decoding of the checkpoint; GEMM output is held to the
same bar as every GEMM (rel-L2 <= 1e-3 fp16 / 4e-3 bf16, max-abs <= 2e-2 * rms) against the float64
oracle of that format."""
import sys

import numpy as np
import pytest

import oracle as o
import gptq_inputs as gi
from gpu_util import bits_to_device, check, check_runtime_perm, run_gemm

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


def repack_fmt(L, fmt):
    import torch
    import weight_only_quantized_amd as wq
    qw = torch.from_numpy(np.ascontiguousarray(L.qweight)).cuda()
    qz = torch.from_numpy(np.ascontiguousarray(L.qzeros)).cuda()
    sc = bits_to_device(L.scales, L.scales_dtype)
    g = torch.from_numpy(np.ascontiguousarray(L.g_idx, dtype=np.int32)).cuda()
    return wq.repack(qw, qz, sc, g, bits=L.bits, group_size=L.group_size, desc_act=L.desc_act, checkpoint_format=fmt)


def expected_codes_zeros(L, fmt):
    if fmt == "gptq_p":
        return o.planar_unpack_rows(L.qweight, L.bits), o.planar_unpack_cols(L.qzeros, L.bits) + 1
    return o.unpack_codes(L.qweight, L.bits), o.unpack_along_cols(L.qzeros, L.bits)   # gptq_v2


@pytest.mark.parametrize("fmt,bits,gs,desc,sdt", [
    ("gptq_p", 2, 64, True, "f16"), ("gptq_p", 3, 32, True, "bf16"), ("gptq_p", 4, 128, False, "f16"),
    ("gptq_p", 5, 64, True, "f16"), ("gptq_p", 6, 128, False, "f32"), ("gptq_p", 7, -1, True, "bf16"),
    ("gptq_p", 8, 32, False, "f16"), ("gptq_v2", 2, 64, False, "bf16"), ("gptq_v2", 3, 32, True, "f16"),
    ("gptq_v2", 4, 128, True, "f32"), ("gptq_v2", 8, 64, False, "f16"),
])
def test_repack_decodes_to_the_formats_codes_and_zeros(fmt, bits, gs, desc, sdt):
    K, N = 384, 96
    say("fmt-repack", fmt, bits, gs, desc, sdt)
    L = gi.make_layer(K, N, bits, gs, desc_act=desc, scales_dtype=sdt, seed=K + 17 * bits + gs)
    h = repack_fmt(L, fmt)
    d = h.decode()
    codes, zeros = expected_codes_zeros(L, fmt)
    assert np.array_equal(d["codes"], codes)
    assert np.array_equal(d["zeros"], zeros.astype(np.int32))
    want_sc = L.scales.view(np.uint32) if sdt == "f32" else L.scales.astype(np.uint32)
    assert np.array_equal(d["scales"], want_sc)
    check_runtime_perm(d["perm"], L.g_idx, gs)
    assert h.info()["bits"] == bits
    h.close()


MS = [1, 3, 16, 17, 33, 64, 65, 130]


@pytest.mark.parametrize("fmt,bits,K,gs,desc,sdt,xdt", [
    ("gptq_p", 3, 544, 32, True, "f16", "f16"), ("gptq_p", 5, 384, 128, False, "bf16", "bf16"),
    ("gptq_p", 6, 256, 64, True, "f16", "bf16"), ("gptq_p", 7, 416, -1, False, "f32", "f16"),
    ("gptq_v2", 4, 512, 128, True, "f16", "bf16"), ("gptq_v2", 3, 288, 32, False, "bf16", "f16"),
    ("gptq_p", 5, 4096, 128, False, "f16", "f16"), ("gptq_p", 3, 4096, 128, True, "bf16", "bf16"),
    ("gptq_v2", 4, 8192, 128, False, "f16", "bf16"),
])
def test_gemm_formats_every_family(fmt, bits, K, gs, desc, sdt, xdt):
    import weight_only_quantized_amd as wq
    N = 160
    say("fmt-gemm", fmt, bits, K, gs, desc, sdt, xdt)
    L = gi.make_layer(K, N, bits, gs, desc_act=desc, scales_dtype=sdt, seed=3 * K + bits)
    h = repack_fmt(L, fmt)
    x = gi.make_x(max(MS), K, xdt, seed=K + bits)
    y_ref = o.gemm_fmt(fmt, x, xdt, L.qweight, L.qzeros, L.scales, sdt, L.g_idx, bits)
    for M in MS:
        for p in [wq.PATH_AUTO, wq.PATH_TILED] + ([wq.PATH_SKINNY] if M <= 64 else []):
            check(run_gemm(h, x[:M], xdt, path=p), xdt, y_ref[:M], label=(fmt, bits, M, p))
    h.close()


# 5/6/7-bit planar layers in their own runtime widths, on every form the dispatcher has for them:
# the M = 1 rule at 4 / 8 chunks a wave (and 8 where 4-bit codes would take 16), act-order M = 1,
# staged x, x from L2, two row blocks, the 40-chunk waves, 32-input groups, the mid kernel and
# both tiled tiles.
@pytest.mark.parametrize("bits,K,gs,desc,sdt,xdt", [
    (5, 4096, 128, False, "f16", "bf16"), (6, 8192, 128, True, "f16", "f16"), (7, 8192, 128, False, "bf16", "bf16"),
    (6, 10240, 128, False, "f16", "f16"), (7, 14336, -1, False, "f32", "f16"), (5, 5120, 128, False, "bf16", "f16"),
    (7, 2048, 32, True, "f16", "bf16"), (6, 16384, 128, False, "f16", "bf16"), (5, 8192, 256, True, "bf16", "bf16"),
])
def test_native_wide_codes_every_form(bits, K, gs, desc, sdt, xdt):
    import weight_only_quantized_amd as wq
    N = 256
    say("wide-codes", bits, K, gs, desc, sdt, xdt)
    L = gi.make_layer(K, N, bits, gs, desc_act=desc, scales_dtype=sdt, seed=7 * K + bits)
    h = repack_fmt(L, "gptq_p")
    assert h.info()["bits"] == bits
    rows = [1, 2, 3, 5, 8, 12, 16, 17, 24, 33, 64, 65, 130]
    x = gi.make_x(max(rows), K, xdt, seed=K + 3 * bits)
    y_ref = o.gemm_fmt("gptq_p", x, xdt, L.qweight, L.qzeros, L.scales, sdt, L.g_idx, bits)
    for M in rows:
        for p in [wq.PATH_AUTO, wq.PATH_TILED] + ([wq.PATH_SKINNY] if M <= 64 else []):
            check(run_gemm(h, x[:M], xdt, path=p), xdt, y_ref[:M], label=("wide", bits, K, M, p))
    h.close()


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_v2_zero_of_zero(xdt):
    """A v2 zero of 0 (which v1 cannot store) on every family: W = code * scale there."""
    import weight_only_quantized_amd as wq
    K, N, bits, gs = 2048, 64, 4, 128
    base = gi.make_layer(K, N, bits, gs, seed=55)
    zeros = np.zeros((K // gs, N), dtype=np.int64)
    zeros[:, ::2] = 15
    L = gi.Layer(K, N, bits, gs, False, base.qweight, o.pack_along_cols(zeros, bits), base.scales, "f16", base.g_idx)
    h = repack_fmt(L, "gptq_v2")
    assert np.array_equal(h.decode()["zeros"], zeros.astype(np.int32))
    x = gi.make_x(130, K, xdt, seed=56)
    y_ref = o.gemm_fmt("gptq_v2", x, xdt, L.qweight, L.qzeros, L.scales, "f16", L.g_idx, bits)
    for M in (1, 5, 40, 130):
        for p in [wq.PATH_AUTO, wq.PATH_TILED] + ([wq.PATH_SKINNY] if M <= 64 else []):
            check(run_gemm(h, x[:M], xdt, path=p), xdt, y_ref[:M], label=(M, p))
    h.close()


def test_formats_refused_where_the_encoding_cannot_hold_the_layer():
    import torch
    import weight_only_quantized_amd as wq
    L = gi.make_layer(256, 64, 6, 64, seed=3)
    qw = torch.from_numpy(L.qweight).cuda()
    qz = torch.from_numpy(L.qzeros).cuda()
    sc = bits_to_device(L.scales, "f16")
    for fmt in ("gptq", "gptq_v2"):          # 6-bit codes exist only as planar words
        with pytest.raises(wq.GPTQError) as e:
            wq.repack(qw, qz, sc, None, bits=6, group_size=64, checkpoint_format=fmt)
        assert e.value.name == "E_UNSUPPORTED"
    h = wq.repack(qw, qz, sc, None, bits=6, group_size=64, checkpoint_format="gptq_p")
    assert h.info()["bits"] == 6
    h.close()
