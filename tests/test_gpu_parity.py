"""GPU parity: the HIP path against the float64 CPU oracle, element by element, through the C ABI.

Repack must be bit-exact (decoded runtime layout == oracle unpack).  GEMM output must be within
rel-L2 <= 1e-3 (fp16 out) / 4e-3 (bf16 out) and max-abs <= 2e-2 * rms(y_ref).  Cases with a
single nonzero product per output must be bit-exact."""
import itertools
import os
import sys

import numpy as np
import pytest

import oracle as o
import gptq_inputs as gi
from gpu_util import TOL, bits_to_device, check, check_runtime_perm, device_to_bits, repack_layer, run_gemm, torch_dtype

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


# ---- repack: bit-exact ---------------------------------------------------------------------------

REPACK_CASES = [
    (256, 256, 4, 128, False, "f16"), (256, 96, 2, 64, True, "bf16"), (288, 64, 3, 32, True, "f16"),
    (512, 64, 8, -1, True, "f32"), (96, 32, 4, 32, False, "bf16"), (1024, 160, 3, 128, True, "f16"),
    (384, 64, 8, 96, True, "f16"), (4096, 128, 4, 128, True, "f16"),
]


@pytest.mark.parametrize("K,N,bits,gs,desc,sdt", REPACK_CASES)
def test_repack_decodes_to_oracle_unpack(K, N, bits, gs, desc, sdt):
    say("repack", K, N, bits, gs, desc, sdt)
    L = gi.make_layer(K, N, bits, gs, desc_act=desc, scales_dtype=sdt, seed=K + N + bits)
    h = repack_layer(L)
    d = h.decode()
    assert np.array_equal(d["codes"], o.unpack_codes(L.qweight, bits))
    assert np.array_equal(d["zeros"], o.unpack_zeros(L.qzeros, bits))
    want_sc = L.scales.view(np.uint32) if sdt == "f32" else L.scales.astype(np.uint32)
    assert np.array_equal(d["scales"], want_sc)
    check_runtime_perm(d["perm"], L.g_idx, gs)
    assert h.info()["has_perm"] == int(not np.array_equal(o.runtime_perm(L.g_idx), np.arange(K)))
    h.close()


# ---- GEMM parity on small shapes that span several tiles and a ragged tail -----------------------

def _small_cases():
    rng = np.random.default_rng(1234)
    cases = []
    for bits, xdt in itertools.product([2, 3, 4, 8], ["f16", "bf16"]):
        for trial in range(3):
            K = int(rng.choice([32, 96, 160, 256, 384, 544]))
            N = int(rng.choice([32, 64, 96, 160, 288]))
            gs = int(rng.choice([32, 64, 128, -1]))
            if gs > K:
                gs = -1
            desc = bool(rng.integers(0, 2))
            sdt = str(rng.choice(["f16", "bf16", "f32"]))
            cases.append((K, N, bits, gs, desc, sdt, xdt))
    return cases


MS = [1, 2, 3, 5, 8, 16, 17, 33, 64, 65, 130]


@pytest.mark.parametrize("K,N,bits,gs,desc,sdt,xdt", _small_cases())
def test_gemm_small_shapes_both_paths(K, N, bits, gs, desc, sdt, xdt):
    import weight_only_quantized_amd as wq
    say("gemm-small", K, N, bits, gs, desc, sdt, xdt)
    L = gi.make_layer(K, N, bits, gs, desc_act=desc, scales_dtype=sdt, seed=7 * K + N)
    h = repack_layer(L)
    x = gi.make_x(max(MS), K, xdt, seed=K * N)
    y_ref_all = o.gemm(x, xdt, L.qweight, L.qzeros, L.scales, sdt, L.g_idx, bits)
    for M in MS:
        paths = [wq.PATH_TILED] + ([wq.PATH_SKINNY] if M <= 64 else [])
        for p in paths:
            y = run_gemm(h, x[:M], xdt, path=p)
            check(y, xdt, y_ref_all[:M], label=(M, p))
    h.close()


# ---- the kernel variants the dispatcher picks at long K ----------------------------------------
# 16, 32 and 64 chunks of K select the straight-line skinny variants (four or two waves per column
# tile, x staged per wave), the x-from-L2 skinny kernel, the split-K mid kernel and both tiled
# tiles; N = 96 leaves a partial 256-column block on the tiled path.

DISPATCH_MS = [1, 2, 3, 4, 5, 16, 17, 33, 64, 130, 257]


@pytest.mark.parametrize("K,bits,gs,desc,xdt", [(14336, 4, 128, False, "f16"), (14336, 4, 128, False, "bf16"),
                                                (12288, 3, 128, False, "bf16"), (10240, 8, -1, False, "f16"),
                                                (14304, 2, -1, False, "bf16"), (14336, 4, 128, True, "f16"),
                                                (12288, 8, 256, False, "bf16"), (10240, 4, 64, False, "f16")])
def test_long_rows_at_one_row(K, bits, gs, desc, xdt):
    """M = 1 on 10240 / 12288 / 14336-input layers: x staged in LDS by ten to fourteen waves of 8
    chunks per column tile (whole-chunk groups, no act-order; 14304 inputs end in a partial chunk);
    M = 2 .. 12: five to seven waves of 16 chunks with x read from L2; act-order and 64-input
    groups take the mid kernel, M = 16 here the tiled family."""
    import weight_only_quantized_amd as wq
    N = 160
    say("long-rows", K, bits, gs, desc, xdt)
    L = gi.make_layer(K, N, bits, gs, desc_act=desc, scales_dtype="f16", seed=K + bits)
    h = repack_layer(L)
    x = gi.make_x(16, K, xdt, seed=K + 7)
    y_ref = o.gemm(x, xdt, L.qweight, L.qzeros, L.scales, "f16", L.g_idx, bits)
    for M in (1, 2, 3, 5, 12, 16):
        for p in (wq.PATH_AUTO, wq.PATH_SKINNY):
            check(run_gemm(h, x[:M], xdt, path=p), xdt, y_ref[:M], label=(K, bits, gs, desc, xdt, M, p))
    h.close()


# K values of the M = 1 rule (waves of 4 chunks up to 32 chunks, of 8 above, as many waves as K
# needs): whole waves (9216: 72 chunks, 9 waves; 16384: 128 chunks, 16 waves), a last wave with
# padding chunks (11008: 86 chunks, 11 waves, 2 padding; 1152: 9 chunks, 3 waves, 3 padding; 16256:
# 127 chunks, 16 waves, 1 padding), a single wave (128 and 384 inputs), ragged K inside the last
# chunk (4000, 9024), every width, both activation dtypes, all scale dtypes.
M1_RULE = [(9216, 4, "bf16", "f16"), (9216, 3, "f16", "bf16"), (11008, 4, "f16", "f16"), (11008, 8, "bf16", "f32"),
           (11008, 2, "bf16", "bf16"), (1152, 4, "bf16", "f16"), (1152, 8, "f16", "f16"), (16384, 4, "bf16", "bf16"),
           (16256, 3, "bf16", "f16"), (16256, 8, "f16", "bf16"), (128, 4, "f16", "f16"), (384, 2, "bf16", "f32"),
           (4000, 4, "bf16", "f16"), (9024, 8, "f16", "f16"), (4096, 4, "f16", "f16"), (8192, 4, "bf16", "f16")]
# act-order layers at the same K values (x scattered into sorted order in LDS, or a sorted copy of
# x past 8192 inputs)
# act-order at M = 1: the staged form up to 8192 inputs (T = 4 up to 32 chunks, else 16 at 4-bit
# and 8 otherwise; padding chunks at 7936 / 8064 / 1152 / 6144; K = 4000 keeps the stable order),
# the mid kernel beyond
M1_RULE_ACT = [(8192, 2, "f16", "f16"), (8192, 4, "bf16", "f16"), (8192, 8, "f16", "bf16"), (11008, 3, "bf16", "f16"),
               (16384, 4, "f16", "f32"), (1152, 4, "bf16", "bf16"), (4000, 8, "bf16", "f16"), (4096, 4, "f16", "f16"),
               (8192, 3, "bf16", "f32"), (6144, 3, "f16", "f32"), (8064, 2, "bf16", "f16"), (7936, 4, "f16", "bf16"),
               (256, 8, "f16", "f16"), (2048, 2, "f16", "f16"), (7936, 8, "bf16", "f16")]


@pytest.mark.parametrize("K,bits,xdt,sdt,desc", [c + (False,) for c in M1_RULE] + [c + (True,) for c in M1_RULE_ACT])
def test_m1_rule_any_k(K, bits, xdt, sdt, desc):
    """M = 1 through the rule's launch-set K split: one column tile per workgroup, ceil(KC / T)
    waves of T straight-line chunks, padding chunks past the layer (act-order layers: the same K
    values on their own path); checked against the oracle."""
    import weight_only_quantized_amd as wq
    N = 224
    say("m1-rule", K, bits, xdt, sdt, desc)
    L = gi.make_layer(K, N, bits, 128, desc_act=desc, scales_dtype=sdt, seed=K + 3 * bits)
    h = repack_layer(L)
    x = gi.make_x(1, K, xdt, seed=K + 11)
    y_ref = o.gemm(x, xdt, L.qweight, L.qzeros, L.scales, sdt, L.g_idx, bits)
    for p in (wq.PATH_AUTO, wq.PATH_SKINNY):
        check(run_gemm(h, x, xdt, path=p), xdt, y_ref, label=(K, bits, xdt, sdt, desc, p))
    assert h.info()["has_perm"] == int(desc)
    if desc:
        check_runtime_perm(h.decode()["perm"], L.g_idx, 128)
    h.close()


# 2 <= M <= 16 through the copy form (x[0:M] copied into LDS once per workgroup, or in two halves
# of the inputs, column groups and launch-set waves of T chunks, padding chunks past the layer; bf16
# x in the offset form): the shapes pick T = 16 or 32, one or several column groups, one or two
# workgroups per compute unit, padding (24, 9 and 63 chunks), whole-layer and 256-input groups,
# every scale dtype, 2/3/4-bit codes
COPY_FORM = [(8192, 2048, 4, 128, "bf16", "f16", (2, 3, 5, 8)), (8192, 3072, 2, 128, "bf16", "bf16", (4, 7)),
             (8192, 2048, 3, 256, "bf16", "f32", (2, 6)), (4096, 1024, 4, 128, "f16", "f16", (4, 9, 16)),
             (4096, 2048, 3, -1, "bf16", "f16", (12, 16)), (14336, 512, 4, 128, "f16", "bf16", (2, 4)),
             (3072, 512, 4, 128, "f16", "f16", (8, 13)), (1152, 768, 2, 128, "bf16", "f16", (6, 16)),
             (16384, 512, 4, 128, "bf16", "f16", (3, 4)),
             # x copied in two halves of the inputs (the whole rows do not fit the LDS)
             (8192, 2048, 4, 128, "bf16", "f16", (9, 16)), (8192, 1536, 2, 128, "bf16", "bf16", (12,)),
             (14336, 512, 4, 128, "f16", "f16", (5, 8)), (16384, 512, 3, 256, "bf16", "f32", (8, 11)),
             (8064, 1024, 4, 128, "f16", "f16", (16,)),
             # two 16-row blocks (17 <= M <= 32) in one, two or four copy phases
             (8192, 2048, 4, 128, "bf16", "f16", (17, 24, 32)), (4096, 1024, 3, 128, "f16", "bf16", (20, 32)),
             (2048, 768, 2, 128, "bf16", "f32", (32,)), (8192, 1024, 3, -1, "bf16", "f16", (29,))]


@pytest.mark.parametrize("K,N,bits,gs,xdt,sdt,Ms", COPY_FORM)
def test_copy_form(K, N, bits, gs, xdt, sdt, Ms):
    """The copy form against the oracle at each M, on PATH_AUTO and PATH_SKINNY, and with a bias."""
    import weight_only_quantized_amd as wq
    say("copy-form", K, N, bits, gs, xdt, sdt, Ms)
    L = gi.make_layer(K, N, bits, gs, desc_act=False, scales_dtype=sdt, seed=K + N + bits)
    h = repack_layer(L)
    x = gi.make_x(max(Ms), K, xdt, seed=K + 5)
    y_ref = o.gemm(x, xdt, L.qweight, L.qzeros, L.scales, sdt, L.g_idx, bits)
    bias = gi.make_bias(N, sdt, seed=N + 1)
    y_ref_b = y_ref + o.decode_float_bits(bias, sdt)[None, :]
    for M in Ms:
        for p in (wq.PATH_AUTO, wq.PATH_SKINNY):
            check(run_gemm(h, x[:M], xdt, path=p), xdt, y_ref[:M], label=(K, N, bits, gs, xdt, sdt, M, p))
        check(run_gemm(h, x[:M], xdt, bias=bias, bias_tag=sdt), xdt, y_ref_b[:M], label=("bias", K, N, M))
    h.close()


@pytest.mark.parametrize("K,N,bits,xdt,Ms", [(8192, 1024, 2, "f16", (2, 8, 16, 32)), (8192, 768, 4, "bf16", (5, 12, 24)),
                                              (4096, 1024, 3, "bf16", (3, 17, 32))])
def test_copy_form_act_order(K, N, bits, xdt, Ms):
    """Act-order at 2 <= M <= 32: x sorted into the workspace, then the copy form; the oracle
    multiplies x as given against the act-order layer."""
    import weight_only_quantized_amd as wq
    say("copy-form act-order", K, N, bits, xdt, Ms)
    L = gi.make_layer(K, N, bits, 128, desc_act=True, scales_dtype="f16", seed=K + N + 7 * bits)
    h = repack_layer(L)
    assert h.info()["has_perm"] == 1
    x = gi.make_x(max(Ms), K, xdt, seed=K + 9)
    y_ref = o.gemm(x, xdt, L.qweight, L.qzeros, L.scales, "f16", L.g_idx, bits)
    for M in Ms:
        for p in (wq.PATH_AUTO, wq.PATH_SKINNY):
            check(run_gemm(h, x[:M], xdt, path=p), xdt, y_ref[:M], label=("act", K, N, bits, xdt, M, p))
    h.close()


@pytest.mark.parametrize("K,bits,xdt", [(10240, 4, "bf16"), (10240, 3, "f16"), (10240, 8, "bf16"),
                                         (5120, 4, "f16"), (7168, 2, "bf16")])
def test_long_rows_wide_layer(K, bits, xdt):
    """10240 / 5120 / 7168 inputs x 8192 outputs (512 column tiles: two tiles per wave with x from
    L2) at M = 1 .. 16, checked on 256 columns at each end of the layer against the oracle on those
    columns (the packed tensors sliced on whole words)."""
    import weight_only_quantized_amd as wq
    N = 8192
    say("long-rows-wide", bits, xdt)
    L = gi.make_layer(K, N, bits, 128, scales_dtype="f16", seed=K + bits)
    h = repack_layer(L)
    x = gi.make_x(16, K, xdt, seed=K + 9)
    zc = N * bits // 32                              # qzeros words per group row
    refs = []
    for c0 in (0, N - 256):
        wq_cols = L.qweight[:, c0:c0 + 256]
        qz_cols = L.qzeros[:, c0 * bits // 32:(c0 + 256) * bits // 32]
        sc_cols = L.scales[:, c0:c0 + 256]
        refs.append((c0, o.gemm(x, xdt, wq_cols, qz_cols, sc_cols, "f16", L.g_idx, bits)))
    assert zc * 32 == N * bits
    for M in (1, 2, 4, 9, 16):
        for p in (wq.PATH_AUTO, wq.PATH_SKINNY):
            y = run_gemm(h, x[:M], xdt, path=p)
            for c0, yr in refs:
                check(y[:, c0:c0 + 256], xdt, yr[:M], label=(bits, xdt, M, p, c0))
    h.close()


@pytest.mark.parametrize("K,bits,desc,xdt", [(2048, 4, False, "f16"), (4096, 4, False, "f16"),
                                             (4096, 4, False, "bf16"), (4096, 2, False, "f16"),
                                             (4096, 3, False, "bf16"), (4096, 8, False, "f16"),
                                             (8192, 4, False, "f16"), (8192, 4, False, "bf16"),
                                             (4096, 8, False, "bf16"), (8192, 2, False, "bf16"),
                                             (4096, 4, True, "f16"), (8192, 3, True, "bf16"),
                                             (5120, 4, False, "bf16"), (6144, 3, False, "f16"),
                                             (7168, 8, False, "bf16"), (5120, 2, False, "f16"),
                                             (3072, 4, False, "bf16")])
def test_gemm_dispatch_variants(K, bits, desc, xdt):
    import weight_only_quantized_amd as wq
    N = 96
    say("dispatch-variants", K, bits, desc, xdt)
    L = gi.make_layer(K, N, bits, 128, desc_act=desc, scales_dtype="f16", seed=K + 10 * bits + desc)
    h = repack_layer(L)
    x = gi.make_x(max(DISPATCH_MS), K, xdt, seed=K * 3 + bits)
    y_ref_all = o.gemm(x, xdt, L.qweight, L.qzeros, L.scales, "f16", L.g_idx, bits)
    for M in DISPATCH_MS:
        paths = [wq.PATH_AUTO] + ([wq.PATH_SKINNY] if M <= 64 else [])
        for p in paths:
            y = run_gemm(h, x[:M], xdt, path=p)
            check(y, xdt, y_ref_all[:M], label=(K, bits, desc, xdt, M, p))
    h.close()


def test_bf16_rows_longer_than_the_one_pass_prep():
    """bf16 rows of more than 16384 inputs take the two-pass prep; 129 chunks is an odd count."""
    import weight_only_quantized_amd as wq
    K, N = 16512, 256
    say("bf16-long-rows", K, N)
    L = gi.make_layer(K, N, 4, 128, scales_dtype="bf16", seed=5)
    h = repack_layer(L)
    x = gi.make_x(257, K, "bf16", seed=6)
    y_ref_all = o.gemm(x, "bf16", L.qweight, L.qzeros, L.scales, "bf16", L.g_idx, 4)
    for M in (1, 130, 257):
        y = run_gemm(h, x[:M], "bf16", path=wq.PATH_TILED)
        check(y, "bf16", y_ref_all[:M], label=("long-rows", M))
    h.close()


# ---- the layer's optional bias (gptq_gemm_bias) ---------------------------------------------------
# Every family adds the bias in its own epilogue: the skinny kernel (x in LDS, the bf16 M = 1 form,
# x from L2, the copy form), the mid kernel without and with split K (in-kernel store, reduction
# kernel), and both tiled tiles.

BIAS_MS = [1, 3, 8, 17, 33, 130, 257]


@pytest.mark.parametrize("K,sdt,xdt", [(512, "f16", "f16"), (512, "bf16", "bf16"), (4096, "f16", "bf16"),
                                       (4096, "bf16", "bf16"), (4096, "f32", "f16"), (8192, "f16", "bf16")])
def test_gemm_bias_all_families(K, sdt, xdt):
    import weight_only_quantized_amd as wq
    N = 96
    say("gemm-bias", K, sdt, xdt)
    L = gi.make_layer(K, N, 4, 128, scales_dtype=sdt, seed=K + 3)
    h = repack_layer(L)
    bias = gi.make_bias(N, sdt, seed=K + 4)
    x = gi.make_x(max(BIAS_MS), K, xdt, seed=K + 5)
    y_ref_all = o.gemm_bias(x, xdt, L.qweight, L.qzeros, L.scales, sdt, L.g_idx, 4, bias)
    for M in BIAS_MS:
        paths = [wq.PATH_AUTO] + ([wq.PATH_SKINNY] if M <= 64 else [])
        for p in paths:
            y = run_gemm(h, x[:M], xdt, path=p, bias=bias, bias_tag=sdt)
            check(y, xdt, y_ref_all[:M], label=("bias", K, sdt, xdt, M, p))
    h.close()


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_bias_on_a_zero_weight(xdt):
    """W = 0: every output is the bias rounded once to x's dtype.  Bit-exact wherever the operands
    are exact; the bf16 skinny and mid kernels carry an operand offset removed in fp32, so there the
    bar is the bf16 tolerance around the same values."""
    import weight_only_quantized_amd as wq
    K, N, bits, gs = 4096, 64, 4, 128
    rng = np.random.default_rng(3)
    zeros = rng.integers(1, 2 ** bits, size=(K // gs, N))
    codes = zeros[np.arange(K) // gs]
    scales = gi.to_f16_bits(np.full((K // gs, N), 0.01))
    L = gi.Layer(K, N, bits, gs, False, o.pack_codes(codes, bits), o.pack_zeros(zeros, bits), scales, "f16",
                 (np.arange(K) // gs).astype(np.int32))
    h = repack_layer(L)
    bias = gi.make_bias(N, "f16", seed=9)
    x = gi.make_x(130, K, xdt, seed=10)
    want = o.round_to_dtype_bits(np.broadcast_to(o.decode_float_bits(bias, "f16"), (130, N)), xdt)
    for M, p in [(1, wq.PATH_SKINNY), (17, wq.PATH_SKINNY), (64, wq.PATH_SKINNY), (1, wq.PATH_TILED),
                 (130, wq.PATH_TILED)]:
        y = run_gemm(h, x[:M], xdt, path=p, bias=bias, bias_tag="f16")
        if xdt == "f16" or p == wq.PATH_TILED:
            assert np.array_equal(y, want[:M]), (M, p)
        else:
            check(y, xdt, np.broadcast_to(o.decode_float_bits(bias, "f16"), (M, N)), label=(M, p))
    h.close()


def test_bias_null_is_gemm_and_bad_bias_is_rejected():
    import torch
    import weight_only_quantized_amd as wq
    from gpu_util import torch_dtype
    K, N = 512, 64
    L = gi.make_layer(K, N, 4, 128, scales_dtype="f16", seed=21)
    h = repack_layer(L)
    lib = wq.load_library()
    x = bits_to_device(gi.make_x(5, K, "f16", seed=22), "f16")
    y0 = h.gemm(x)
    y1 = torch.empty_like(y0)
    st = lib.gptq_gemm_bias(h.ptr, x.data_ptr(), 5, 0, None, y1.data_ptr(), None, 0, 0, None)
    torch.cuda.synchronize()
    assert st == 0 and torch.equal(y0, y1)
    b = torch.zeros(N + 1, dtype=torch.float16, device="cuda")
    odd = b.data_ptr() + 1                                   # not 2-byte aligned
    assert lib.gptq_gemm_bias(h.ptr, x.data_ptr(), 5, 0, odd, y1.data_ptr(), None, 0, 0, None) == 1
    assert lib.gptq_gemm_bias(h.ptr, x.data_ptr(), 5, 0, y1.data_ptr(), y1.data_ptr(), None, 0, 0, None) == 1
    with pytest.raises(TypeError):
        h.gemm(x, bias=torch.zeros(N, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    h.close()


# ---- closed-form special cases: bit-exact ------------------------------------------------------

@pytest.mark.parametrize("bits,xdt", [(4, "f16"), (4, "bf16"), (2, "f16"), (3, "bf16"), (8, "f16"), (8, "bf16")])
def test_identity_weight(bits, xdt):
    """W = 0.5 * I.  Exact operands make each output one exact product, so it must be bit-exact:
    fp16 activations, 8-bit codes, and the tiled path (which runs bf16 activations as exactly
    rescaled fp16).  The skinny path's 2/3/4-bit bf16 operand carries a constant bias of 144 that
    is removed in fp32 (see dequant.h), so there the bar is the bf16 tolerance."""
    import torch
    import weight_only_quantized_amd as wq
    K = N = 256
    z = 1
    codes = np.full((K, N), z) + np.eye(K, dtype=np.int64)
    zeros = np.full((1, N), z)
    scales = gi.to_f16_bits(np.full((1, N), 0.5))
    L = gi.Layer(K, N, bits, -1, False, o.pack_codes(codes, bits), o.pack_zeros(zeros, bits), scales, "f16",
                 np.zeros(K, dtype=np.int32))
    h = repack_layer(L)
    x = gi.make_x(130, K, xdt, seed=3)
    want = o.round_to_dtype_bits(o.decode_float_bits(x, xdt) * 0.5, xdt)
    for M, p in [(1, wq.PATH_SKINNY), (16, wq.PATH_SKINNY), (64, wq.PATH_SKINNY), (1, wq.PATH_TILED), (130, wq.PATH_TILED)]:
        y = run_gemm(h, x[:M], xdt, path=p)
        if xdt == "f16" or bits == 8 or p == wq.PATH_TILED:
            assert np.array_equal(y, want[:M]), (M, p)
        else:
            check(y, xdt, o.decode_float_bits(x[:M], xdt) * 0.5, label=(M, p))
    h.close()


@pytest.mark.parametrize("K,desc", [(320, False), (512, True)])
def test_bf16_rows_of_extreme_magnitude(K, desc):
    """bf16 activations span 2^-126 .. 2^127; rows scaled by 2^-100 .. 2^100 (and an all-zero row)
    must each stay within tolerance of the oracle, row by row, on both paths."""
    import weight_only_quantized_amd as wq
    N, bits, gs = 192, 4, 64
    say("bf16-extreme-rows", K, desc)
    L = gi.make_layer(K, N, bits, gs, desc_act=desc, scales_dtype="bf16", seed=31 + K)
    h = repack_layer(L)
    M = 130
    xf = o.decode_float_bits(gi.make_x(M, K, "bf16", seed=32 + K), "bf16")
    exps = np.array([-100, -40, 0, 40, 100])[np.arange(M) % 5]
    xf = xf * np.ldexp(1.0, exps)[:, None]
    xf[7] = 0.0
    x = o.round_to_dtype_bits(xf, "bf16")
    assert np.array_equal(o.decode_float_bits(x, "bf16"), xf)       # the scaling itself is exact
    y_ref = o.gemm(x, "bf16", L.qweight, L.qzeros, L.scales, "bf16", L.g_idx, bits)
    for Mc, p in [(M, wq.PATH_TILED), (64, wq.PATH_TILED), (40, wq.PATH_SKINNY), (3, wq.PATH_SKINNY)]:
        y = run_gemm(h, x[:Mc], "bf16", path=p)
        if Mc > 7:
            assert np.all((y[7] & 0x7FFF) == 0), p
        for r in range(Mc):
            if r == 7:
                continue
            check(y[r:r + 1], "bf16", y_ref[r:r + 1], label=(Mc, p, r, int(exps[r])))
    h.close()


def test_zero_weight_gives_exact_zero():
    import weight_only_quantized_amd as wq
    K, N, bits, gs = 256, 64, 4, 64
    rng = np.random.default_rng(2)
    zeros = rng.integers(1, 16, size=(K // gs, N))
    codes = zeros[np.arange(K) // gs]
    L0 = gi.make_layer(K, N, bits, gs, seed=4)
    L = gi.Layer(K, N, bits, gs, False, o.pack_codes(codes, bits), o.pack_zeros(zeros, bits), L0.scales, "f16",
                 L0.g_idx)
    h = repack_layer(L)
    x = gi.make_x(80, K, "f16", seed=5)
    for M, p in [(1, wq.PATH_SKINNY), (80, wq.PATH_TILED)]:
        y = run_gemm(h, x[:M], "f16", path=p)
        assert np.all((y & 0x7FFF) == 0), (M, p)     # fp16 operands are exact zeros
    h.close()


# ---- lifetime and API behaviour -----------------------------------------------------------------

def test_repeated_calls_are_bitwise_identical_and_inputs_can_be_freed():
    import torch
    import weight_only_quantized_amd as wq
    L = gi.make_layer(512, 256, 4, 128, desc_act=True, seed=9)
    h = repack_layer(L)        # the device copies of the checkpoint tensors are dropped right here
    torch.cuda.empty_cache()
    x = bits_to_device(gi.make_x(70, 512, "f16", seed=10), "f16")
    for M, p in [(3, wq.PATH_SKINNY), (70, wq.PATH_TILED)]:
        ys = [device_to_bits(h.gemm(x[:M], path=p)) for _ in range(4)]
        for y in ys[1:]:
            assert np.array_equal(ys[0], y)
    h2 = repack_layer(L)
    assert np.array_equal(device_to_bits(h2.gemm(x[:5])), device_to_bits(h.gemm(x[:5])))
    h.close()
    h2.close()


def test_m_zero_launches_nothing_and_leaves_y_untouched():
    import torch
    import weight_only_quantized_amd as wq
    L = gi.make_layer(256, 64, 4, 128, seed=1)
    h = repack_layer(L)
    lib = wq.load_library()
    y = torch.full((1, 64), 7.0, dtype=torch.float16, device="cuda")
    x = torch.zeros((1, 256), dtype=torch.float16, device="cuda")
    st = lib.gptq_gemm(h.ptr, x.data_ptr(), 0, 0, y.data_ptr(), None, 0, 0, None)
    torch.cuda.synchronize()
    assert st == 0 and torch.all(y == 7.0)
    h.close()


def test_gemm_argument_errors():
    import ctypes
    import torch
    import weight_only_quantized_amd as wq
    lib = wq.load_library()
    L = gi.make_layer(256, 64, 4, 128, desc_act=True, seed=1)
    h = repack_layer(L)
    x = torch.zeros((130, 256), dtype=torch.float16, device="cuda")
    y = torch.zeros((130, 64), dtype=torch.float16, device="cuda")
    need = h.workspace_size(130, torch.float16)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    s = None
    assert lib.gptq_gemm(h.ptr, x.data_ptr(), 130, 0, y.data_ptr(), ws.data_ptr(), need - 1, 0, s) == 7
    assert lib.gptq_gemm(h.ptr, x.data_ptr(), 130, 0, y.data_ptr(), None, 0, 0, s) == 7
    assert lib.gptq_gemm(h.ptr, x.data_ptr() + 2, 1, 0, y.data_ptr(), ws.data_ptr(), need, 0, s) == 1
    assert lib.gptq_gemm(h.ptr, x.data_ptr(), 130, 0, y.data_ptr(), ws.data_ptr(), need, wq.PATH_SKINNY, s) == 1
    assert lib.gptq_gemm(h.ptr, x.data_ptr(), 130, 2, y.data_ptr(), ws.data_ptr(), need, 0, s) == 1
    assert lib.gptq_gemm(h.ptr, x.data_ptr(), -1, 0, y.data_ptr(), ws.data_ptr(), need, 0, s) == 1
    assert lib.gptq_gemm(h.ptr, x.data_ptr(), 130, 0, x.data_ptr(), ws.data_ptr(), need, 0, s) == 1
    torch.cuda.synchronize()
    assert torch.all(y == 0)
    h.close()


def test_repack_rejects_bad_layers_on_device():
    import torch
    import weight_only_quantized_amd as wq
    L = gi.make_layer(256, 64, 4, 64, desc_act=True, seed=2)
    qw = torch.from_numpy(L.qweight).cuda()
    qz = torch.from_numpy(L.qzeros).cuda()
    sc = bits_to_device(L.scales, "f16")
    g = L.g_idx.copy(); g[5] = 4
    with pytest.raises(wq.GPTQError) as e:
        wq.repack(qw, qz, sc, torch.from_numpy(g).cuda(), bits=4, group_size=64)
    assert e.value.name == "E_GIDX"
    with pytest.raises(wq.GPTQError) as e:
        wq.repack(qw, qz, sc, torch.from_numpy(L.g_idx).cuda(), bits=4, group_size=64, checkpoint_format="marlin")
    assert e.value.name == "E_UNSUPPORTED"
    with pytest.raises(wq.GPTQError) as e:
        wq.repack(qw[:-1].contiguous(), qz, sc, torch.from_numpy(L.g_idx).cuda(), bits=4, group_size=64)
    assert e.value.name in ("E_SHAPE", "E_GIDX")


# ---- extreme shapes: very long K, very wide N ------------------------------------------------------

@pytest.mark.parametrize("K,N,bits,gs,desc,xdt", [(65536, 64, 4, 128, False, "bf16"), (32768, 96, 3, 128, True, "f16"),
                                                  (128, 131072, 4, -1, False, "f16"), (256, 65536, 8, 128, True, "bf16")])
def test_extreme_shapes(K, N, bits, gs, desc, xdt):
    """512 chunks of K (split K up to its 255-slice cap on the tiled path, long skinny ranges) and
    4096-8192 column tiles; every family."""
    import weight_only_quantized_amd as wq
    say("extreme", K, N, bits, gs, desc, xdt)
    L = gi.make_layer(K, N, bits, gs, desc_act=desc, scales_dtype="f16", seed=K % 9973 + N)
    h = repack_layer(L)
    x = gi.make_x(130, K, xdt, seed=K + N + 1)
    y_ref = o.gemm(x, xdt, L.qweight, L.qzeros, L.scales, "f16", L.g_idx, bits)
    for M in (1, 5, 33, 130):
        for p in [wq.PATH_AUTO, wq.PATH_TILED] + ([wq.PATH_SKINNY] if M <= 64 else []):
            check(run_gemm(h, x[:M], xdt, path=p), xdt, y_ref[:M], label=(K, N, M, p))
    h.close()
