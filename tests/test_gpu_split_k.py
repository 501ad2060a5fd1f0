"""GPU parity of the tiled family's tile table and split K: every tile the plan picks, slices of
unequal length (a ragged chunk count), every width, act-order, 32-input segments, bf16 rows
(multiplied back to scale before the partial sums are stored), the bias added by the reduction,
and bit-exact closed forms through the partial sums.  Same bar as every GEMM: rel-L2 <= 1e-3
(fp16) / 4e-3 (bf16) and max-abs <= 2e-2 * rms against the float64 oracle."""
import sys

import numpy as np
import pytest

import oracle as o
import gptq_inputs as gi
from gpu_util import check, repack_layer, run_gemm

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


# With N = 96..288 the column tiles are few, so the plan splits K as far as it may (four chunks
# per slice at least); M up to 64 takes the 64 x 128 tile, larger M the 128 x 256 tile, and
# group sizes that are not a multiple of 128 the 128 x 128 tile.  K = 2080 has 17 chunks: slices
# of 5, 5, 5 and 2.
SPLIT_MS = [1, 5, 17, 33, 64, 65, 130, 200, 257, 1000]


@pytest.mark.parametrize("K,N,bits,gs,desc,sdt,xdt", [
    (2048, 256, 4, 128, False, "f16", "f16"), (2080, 160, 4, 128, False, "bf16", "bf16"),
    (2048, 96, 3, 64, True, "f16", "bf16"), (4096, 256, 8, 128, True, "bf16", "f16"),
    (2176, 288, 2, 32, False, "f32", "bf16"), (4224, 128, 4, -1, True, "f16", "f16"),
])
def test_tiled_split_k(K, N, bits, gs, desc, sdt, xdt):
    import weight_only_quantized_amd as wq
    say("split-k", K, N, bits, gs, desc, sdt, xdt)
    L = gi.make_layer(K, N, bits, gs, desc_act=desc, scales_dtype=sdt, seed=K + N + bits)
    h = repack_layer(L)
    x = gi.make_x(max(SPLIT_MS), K, xdt, seed=K - N)
    y_ref = o.gemm(x, xdt, L.qweight, L.qzeros, L.scales, sdt, L.g_idx, bits)
    for M in SPLIT_MS:
        for p in (wq.PATH_TILED, wq.PATH_AUTO):
            check(run_gemm(h, x[:M], xdt, path=p), xdt, y_ref[:M], label=(M, p))
    h.close()


@pytest.mark.parametrize("K", [128, 256, 384, 640, 896, 1152, 1664])
def test_two_deep_tile_every_chunk_count(K):
    """The 64 x 128 tile keeps two chunks in flight in steps of three and finishes a slice with
    one or two steps that issue nothing: slices of 1, 2, 3, 5, 7 chunks (one slice), 5 + 4 and
    5 + 5 + 3 chunks (K split), every one against the oracle."""
    import weight_only_quantized_amd as wq
    say("two-deep", K)
    N = 128
    L = gi.make_layer(K, N, 4, 128, scales_dtype="f16", seed=K)
    h = repack_layer(L)
    for xdt in ("f16", "bf16"):
        x = gi.make_x(64, K, xdt, seed=K + 1)
        y_ref = o.gemm(x, xdt, L.qweight, L.qzeros, L.scales, "f16", L.g_idx, 4)
        for M in (17, 40, 64):
            check(run_gemm(h, x[:M], xdt, path=wq.PATH_TILED), xdt, y_ref[:M], label=(K, xdt, M))
    h.close()


@pytest.mark.parametrize("sdt,xdt", [("f16", "f16"), ("bf16", "bf16"), ("f32", "bf16")])
def test_split_k_bias(sdt, xdt):
    import weight_only_quantized_amd as wq
    K, N = 4096, 192
    say("split-k-bias", sdt, xdt)
    L = gi.make_layer(K, N, 4, 128, scales_dtype=sdt, seed=77)
    h = repack_layer(L)
    b = gi.make_bias(N, sdt, seed=78)
    x = gi.make_x(257, K, xdt, seed=79)
    y_ref = o.gemm_bias(x, xdt, L.qweight, L.qzeros, L.scales, sdt, L.g_idx, 4, b)
    for M in (2, 40, 100, 257):
        check(run_gemm(h, x[:M], xdt, path=wq.PATH_TILED, bias=b, bias_tag=sdt), xdt, y_ref[:M], label=M)
    h.close()


def test_split_k_bf16_rows_of_extreme_magnitude():
    """Each slice stores its partial sums already multiplied back by the row's power of two; rows
    scaled by 2^-100 .. 2^100 and an all-zero row stay within tolerance row by row."""
    import weight_only_quantized_amd as wq
    K, N = 2048, 128
    L = gi.make_layer(K, N, 4, 128, scales_dtype="bf16", seed=5)
    h = repack_layer(L)
    M = 130
    xf = o.decode_float_bits(gi.make_x(M, K, "bf16", seed=6), "bf16")
    exps = np.array([-100, -40, 0, 40, 100])[np.arange(M) % 5]
    xf = xf * np.ldexp(1.0, exps)[:, None]
    xf[7] = 0.0
    x = o.round_to_dtype_bits(xf, "bf16")
    y_ref = o.gemm(x, "bf16", L.qweight, L.qzeros, L.scales, "bf16", L.g_idx, 4)
    for Mc in (M, 48):
        y = run_gemm(h, x[:Mc], "bf16", path=wq.PATH_TILED)
        assert np.all((y[7] & 0x7FFF) == 0)
        for r in range(Mc):
            if r != 7:
                check(y[r:r + 1], "bf16", y_ref[r:r + 1], label=(Mc, r, int(exps[r])))
    h.close()


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_split_k_identity_weight_is_exact(xdt):
    """W = 0.5 * I: each output is one exact product in one slice and exact zeros in the others,
    so the sum of the partials, rounded once, must be bit-exact."""
    import weight_only_quantized_amd as wq
    K = N = 2048
    codes = np.full((K, N), 1) + np.eye(K, dtype=np.int64)
    L = gi.Layer(K, N, 4, -1, False, o.pack_codes(codes, 4), o.pack_zeros(np.full((1, N), 1), 4),
                 gi.to_f16_bits(np.full((1, N), 0.5)), "f16", np.zeros(K, dtype=np.int32))
    h = repack_layer(L)
    x = gi.make_x(130, K, xdt, seed=8)
    want = o.round_to_dtype_bits(o.decode_float_bits(x, xdt) * 0.5, xdt)
    for M in (3, 64, 130):
        assert np.array_equal(run_gemm(h, x[:M], xdt, path=wq.PATH_TILED), want[:M]), M
    h.close()


def test_workspace_covers_the_partial_sums():
    """The workspace query grows by the partial sums when the plan splits K, and a call with less
    is refused rather than run."""
    import torch
    import weight_only_quantized_amd as wq
    K, N = 4096, 128
    L = gi.make_layer(K, N, 4, 128, seed=3)
    h = repack_layer(L)
    need = h.workspace_size(64, torch.float16, path=wq.PATH_TILED)
    assert need >= 2 * 64 * N * 4                       # at least two slices of fp32 partials
    x = torch.zeros(64, K, dtype=torch.float16, device="cuda")
    y = torch.empty(64, N, dtype=torch.float16, device="cuda")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    lib = wq.load_library()
    assert lib.gptq_gemm(h.ptr, x.data_ptr(), 64, 0, y.data_ptr(), ws.data_ptr(), need - 256, wq.PATH_TILED,
                         None) == 7                      # GPTQ_E_WORKSPACE
    assert lib.gptq_gemm(h.ptr, x.data_ptr(), 64, 0, y.data_ptr(), ws.data_ptr(), need, wq.PATH_TILED, None) == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0
    h.close()
