"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a hand-written word from the pages' bit-order
rules, the pages' example header, exact rational arithmetic, a closed-form special case or an
invariant of the definition.  All run on the CPU (no GPU marker).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as o
import gptq_inputs as gi

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _u(h):
    return int(h, 16)


# ---- P-1 / P-2: bit positions, from hand-written words ------------------------------------------

def test_hex_words_unpack_to_stated_codes():
    fx = json.load(open(os.path.join(GOLD, "hex_words.json")))
    for row in fx["rows"]:
        b = row["bits"]
        words = np.array([[_u(w)] for w in row["words"]], dtype=np.uint32).view(np.int32)
        codes = o.unpack_codes(words, b)[:, 0]
        if "codes" in row:
            want = np.array(row["codes"])
        else:
            want = np.zeros(32, dtype=np.int64)
            for j, v in row["codes_nonzero"].items():
                want[int(j)] = v
        assert codes.tolist() == want.tolist(), row
        # the writer must produce exactly the hand-written words
        back = o.pack_codes(want.reshape(-1, 1), b)[:, 0].view(np.uint32)
        assert [int(v) for v in back] == [_u(w) for w in row["words"]], row


def test_hex_zero_words():
    fx = json.load(open(os.path.join(GOLD, "hex_words.json")))
    for z in fx["zeros"]:
        b = z["bits"]
        qz = np.array([[_u(z["qzeros_word"])]], dtype=np.uint32).view(np.int32)
        assert o.unpack_zeros(qz, b)[0].tolist() == z["zeros_along_n"]


def test_three_bit_ten_split_ten_structure():
    """'10 / split / 10': codes 0..9 only touch word 0, code 10 straddles words 0/1, codes 11..20
    only touch word 1, code 21 straddles 1/2, codes 22..31 only word 2."""
    for j in range(32):
        c = np.zeros((32, 1), dtype=np.int64)
        c[j] = 7
        w = o.pack_codes(c, 3)[:, 0].view(np.uint32)
        touched = [i for i in range(3) if w[i]]
        want = {10: [0, 1], 21: [1, 2]}.get(j, [0] if j < 10 else [1] if j < 21 else [2])
        assert touched == want, (j, [hex(v) for v in w])
        assert sum(bin(int(v)).count("1") for v in w) == 3


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_every_word_is_valid_and_round_trips(bits):
    rng = np.random.default_rng(bits)
    words = rng.integers(0, 2 ** 32, size=(bits * 4, 7), dtype=np.uint64).astype(np.uint32).view(np.int32)
    codes = o.unpack_codes(words, bits)
    assert codes.shape == (128, 7)
    assert codes.min() >= 0 and codes.max() < 2 ** bits
    assert np.array_equal(o.pack_codes(codes, bits), words)
    c2 = rng.integers(0, 2 ** bits, size=(96, 5))
    assert np.array_equal(o.unpack_codes(o.pack_codes(c2, bits), bits), c2)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_single_hot_fields_are_independent(bits):
    """Changing one code changes exactly one unpacked code, for every position and value."""
    base = np.zeros((32, 1), dtype=np.int64)
    for j in range(32):
        for v in range(1, 2 ** bits, max(1, (2 ** bits - 1) // 5)):
            c = base.copy()
            c[j] = v
            back = o.unpack_codes(o.pack_codes(c, bits), bits)[:, 0]
            assert back[j] == v and np.count_nonzero(back) == 1


# ---- P-3: stored-minus-one zeros ----------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_zero_minus_one_and_wrap(bits):
    z = np.arange(0, 2 ** bits + 1).reshape(1, -1)
    z = np.pad(z, ((0, 0), (0, (-z.shape[1]) % 32)), constant_values=1)
    back = o.unpack_zeros(o.pack_zeros(z, bits), bits)[0]
    for zi, bi in zip(z[0], back):
        if zi == 0:
            assert bi == 2 ** bits            # logical 0 is not representable: reads back as 2**bits
        else:
            assert bi == zi                   # 1 .. 2**bits round-trip exactly


# ---- P-4 / P-7: exact rational brute force ------------------------------------------------------

def _exact_y(x_bits, x_dtype, codes, zeros, scale_bits, s_dtype, g_idx):
    x = o.decode_float_bits(x_bits, x_dtype)
    s = o.decode_float_bits(scale_bits, s_dtype)
    M, K = x.shape
    N = codes.shape[1]
    y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = int(g_idx[k])
                acc += Fraction(float(x[m, k])) * (int(codes[k, n]) - int(zeros[g, n])) * Fraction(float(s[g, n]))
            y[m][n] = acc
    return y


@pytest.mark.parametrize("bits,gs,desc,sdt,xdt", [
    (4, 32, False, "f16", "f16"), (3, 32, True, "bf16", "bf16"), (2, 64, True, "f16", "bf16"),
    (8, -1, False, "f32", "f16"), (4, 64, True, "bf16", "f16"),
])
def test_gemm_matches_exact_rationals(bits, gs, desc, sdt, xdt):
    rng = np.random.default_rng(7 + bits)
    K, N, M = 64, 32, 3
    G = o.num_groups(K, gs)
    codes = rng.integers(0, 2 ** bits, size=(K, N))
    zeros = rng.integers(1, 2 ** bits + 1, size=(G, N))          # the representable range
    scales = gi.make_layer(K, N, bits, gs, scales_dtype=sdt, seed=3).scales
    g_idx = (rng.permutation(K) if desc else np.arange(K)) // (K if gs == -1 else gs)
    x = gi.make_x(M, K, xdt, seed=5)
    qw, qz = o.pack_codes(codes, bits), o.pack_zeros(zeros, bits)
    # dequant is exact in float64
    W = o.dequant(qw, qz, scales, sdt, g_idx, bits)
    s64 = o.decode_float_bits(scales, sdt)
    for n in range(0, N, 7):
        for k in range(0, K, 5):
            g = g_idx[k]
            assert Fraction(float(W[n, k])) == (int(codes[k, n]) - int(zeros[g, n])) * Fraction(float(s64[g, n]))
    y = o.gemm(x, xdt, qw, qz, scales, sdt, g_idx, bits)
    ye = _exact_y(x, xdt, codes, zeros, scales, sdt, g_idx)
    xa = np.abs(o.decode_float_bits(x, xdt))
    bound = 1e-13 * (xa @ np.abs(W.T))
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(y[m, n])) - ye[m][n]) <= Fraction(float(bound[m, n])) + Fraction(1, 10 ** 30)


def test_gemm_entries_agree_with_gemm():
    L = gi.make_layer(256, 96, 3, 64, desc_act=True, seed=11)
    x = gi.make_x(4, 256, "bf16", seed=12)
    y = o.gemm(x, "bf16", L.qweight, L.qzeros, L.scales, "f16", L.g_idx, 3, chunk=40)
    rows, cols = [0, 3, 2, 1, 3], [0, 95, 40, 63, 1]
    e = o.gemm_entries(x, "bf16", L.qweight, L.qzeros, L.scales, "f16", L.g_idx, 3, rows, cols)
    assert np.allclose(e, y[rows, cols], rtol=0, atol=1e-12 * np.abs(y).max())


# ---- P-5: effective bits ------------------------------------------------------------------------

def test_effective_bits_at_group_128():
    for w in gi.WORKLOADS:
        for b in w["bits"]:
            for gs in w["group_sizes"]:
                if b == 4 and gs == 128:
                    assert o.effective_bits(w["K"], w["N"], 4, 128) == 4.125
                    assert o.effective_bits(w["K"], w["N"], 4, 128, with_zeros=True) == 4.15625


# ---- P-6: the example header and the reject rules -----------------------------------------------

def test_example_header_validates_and_mutations_are_rejected():
    h = json.load(open(os.path.join(GOLD, "small_gptq_header.json")))
    t = h["tensors"]
    qw, qz, sc, gi_ = (t["gptq.qweight"]["shape"], t["gptq.qzeros"]["shape"], t["gptq.scales"]["shape"],
                       t["gptq.g_idx"]["shape"])
    K, N, bits = gi_[0], qw[1], 4
    assert qw[0] == K // 32 * bits
    G = qz[0]
    gs = K // G
    assert (K, N, G, gs) == (256, 32, 8, 32) == (h["implied"]["in_features"], h["implied"]["out_features"],
                                                 h["implied"]["groups"], h["implied"]["group_size"])
    # byte accounting of the container: element size x count fills each data range exactly
    for name, e in t.items():
        n = int(np.prod(e["shape"]))
        assert e["data_offsets"][1] - e["data_offsets"][0] == 4 * n, name
    g = np.arange(K) // gs
    assert o.validate_layer(K, N, bits, gs, qw, qz, sc, g) == "ok"
    assert o.validate_layer(K, N, 5, gs, qw, qz, sc, g) == "unsupported"                 # GPTQ-001
    assert o.validate_layer(K, N, bits, gs, [31, 32], qz, sc, g) == "shape"               # GPTQ-002
    assert o.validate_layer(K - 16, N, bits, gs, qw, qz, sc, g[:-16]) == "shape"          # GPTQ-002
    assert o.validate_layer(K, N, bits, gs, qw, [8, 5], sc, g) == "shape"                 # GPTQ-003
    bad = g.copy(); bad[3] = G
    assert o.validate_layer(K, N, bits, gs, qw, qz, sc, bad) == "gidx"                     # GPTQ-004
    bad[3] = -1
    assert o.validate_layer(K, N, bits, gs, qw, qz, sc, bad) == "gidx"
    assert o.validate_layer(K, N, bits, gs, qw, qz, sc, g, checkpoint_format="marlin") == "unsupported"  # GPTQ-005
    uneven = g.copy(); uneven[0] = 1                                                     # group 0 short, 1 long
    assert o.validate_layer(K, N, bits, gs, qw, qz, sc, uneven) == "unsupported"
    assert o.validate_layer(K, N, bits, 48, qw, [6, 4], [6, 32], None) == "unsupported"   # gs not multiple of 32


# ---- P-8: special cases with closed-form results ------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_code_equal_zero_gives_zero_output(bits):
    rng = np.random.default_rng(bits)
    K, N, gs = 128, 64, 32
    G = K // gs
    zeros = rng.integers(1, 2 ** bits, size=(G, N))
    codes = zeros[np.arange(K) // gs]
    L = gi.make_layer(K, N, bits, gs, seed=1)
    y = o.gemm(gi.make_x(3, K, "f16", seed=2), "f16", o.pack_codes(codes, bits), o.pack_zeros(zeros, bits),
               L.scales, "f16", L.g_idx, bits)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("sdt", ["f16", "bf16", "f32"])
def test_bias_on_a_zero_weight_is_the_output(sdt):
    """code == zero everywhere: W = 0, so every output row is the bias itself, decoded from the
    scales' dtype ([SPEC] GptqLayer bias)."""
    rng = np.random.default_rng(11)
    K, N, gs, bits = 128, 64, 64, 4
    G = K // gs
    zeros = rng.integers(1, 2 ** bits, size=(G, N))
    codes = zeros[np.arange(K) // gs]
    L = gi.make_layer(K, N, bits, gs, scales_dtype=sdt, seed=4)
    bias = gi.make_bias(N, sdt, seed=5)
    y = o.gemm_bias(gi.make_x(3, K, "bf16", seed=6), "bf16", o.pack_codes(codes, bits), o.pack_zeros(zeros, bits),
                    L.scales, sdt, L.g_idx, bits, bias)
    want = o.decode_float_bits(bias, sdt)
    assert np.all(np.isfinite(want)) and np.any(want != 0)
    assert np.array_equal(y, np.broadcast_to(want, y.shape))


@pytest.mark.parametrize("bits,sdt,xdt", [(4, "f16", "f16"), (3, "bf16", "bf16"), (8, "f32", "f16")])
def test_gemm_bias_matches_exact_rationals(bits, sdt, xdt):
    rng = np.random.default_rng(17 + bits)
    K, N, M, gs = 64, 32, 3, 32
    G = o.num_groups(K, gs)
    codes = rng.integers(0, 2 ** bits, size=(K, N))
    zeros = rng.integers(1, 2 ** bits + 1, size=(G, N))
    scales = gi.make_layer(K, N, bits, gs, scales_dtype=sdt, seed=3).scales
    g_idx = np.arange(K) // gs
    x = gi.make_x(M, K, xdt, seed=5)
    bias = gi.make_bias(N, sdt, seed=8)
    qw, qz = o.pack_codes(codes, bits), o.pack_zeros(zeros, bits)
    y = o.gemm_bias(x, xdt, qw, qz, scales, sdt, g_idx, bits, bias)
    ye = _exact_y(x, xdt, codes, zeros, scales, sdt, g_idx)
    b = o.decode_float_bits(bias, sdt)
    W = o.dequant(qw, qz, scales, sdt, g_idx, bits)
    bound = 1e-13 * (np.abs(o.decode_float_bits(x, xdt)) @ np.abs(W.T) + np.abs(b)[None, :])
    for m in range(M):
        for n in range(N):
            exact = ye[m][n] + Fraction(float(b[n]))
            assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(float(bound[m, n])) + Fraction(1, 10 ** 30)


@pytest.mark.parametrize("bits,p", [(2, 3), (4, 5), (8, 1), (3, 0)])
def test_identity_weight_gives_scaled_x(bits, p):
    K = N = 64
    z = 1
    codes = np.full((K, N), z) + np.eye(K, dtype=np.int64)         # W = (c - z) * s = s * I
    zeros = np.full((1, N), z)
    scales = gi.to_f16_bits(np.full((1, N), 2.0 ** -p))
    x = gi.make_x(5, K, "f16", seed=9)
    y = o.gemm(x, "f16", o.pack_codes(codes, bits), o.pack_zeros(zeros, bits), scales, "f16",
               np.zeros(K, dtype=np.int32), bits)
    assert np.array_equal(y, o.decode_float_bits(x, "f16") * 2.0 ** -p)


def test_single_nonzero_column():
    K, N, bits = 64, 32, 4
    zeros = np.full((2, N), 8)
    codes = np.full((K, N), 8)
    codes[:, 5] = np.arange(K) % 16
    scales = gi.to_f16_bits(np.full((2, N), 0.25))
    x = gi.make_x(2, K, "f16", seed=4)
    y = o.gemm(x, "f16", o.pack_codes(codes, bits), o.pack_zeros(zeros, bits), scales, "f16", np.arange(K) // 32, bits)
    xf = o.decode_float_bits(x, "f16")
    assert np.all(np.delete(y, 5, axis=1) == 0)
    assert np.allclose(y[:, 5], xf @ ((np.arange(K) % 16 - 8) * 0.25), rtol=1e-15, atol=0)


# ---- P-9: invariants -----------------------------------------------------------------------------

@pytest.mark.parametrize("bits,gs", [(4, 128), (3, 64), (2, 32), (8, 128)])
def test_act_order_equals_sorted_sequential_layer(bits, gs):
    K, N = 256, 64
    L = gi.make_layer(K, N, bits, gs, desc_act=True, seed=21)
    x = gi.make_x(3, K, "f16", seed=22)
    y = o.gemm(x, "f16", L.qweight, L.qzeros, L.scales, "f16", L.g_idx, bits)
    perm = o.runtime_perm(L.g_idx)
    assert np.array_equal(L.g_idx[perm], np.arange(K) // gs)
    codes = o.unpack_codes(L.qweight, bits)[perm]
    y2 = o.gemm(x[:, perm], "f16", o.pack_codes(codes, bits), L.qzeros, L.scales, "f16", np.arange(K) // gs, bits)
    assert np.allclose(y, y2, rtol=0, atol=1e-12 * np.abs(y).max())
    # and a wrong group map (ignoring g_idx) would differ
    y3 = o.gemm(x, "f16", L.qweight, L.qzeros, L.scales, "f16", np.arange(K) // gs, bits)
    assert not np.allclose(y, y3, rtol=0, atol=1e-6 * np.abs(y).max())


def test_runtime_perm_is_stable():
    g = np.array([2, 0, 1, 0, 2, 1, 0, 1])
    assert o.runtime_perm(g).tolist() == [1, 3, 6, 2, 5, 7, 0, 4]
    assert o.runtime_perm(np.arange(64) // 32).tolist() == list(range(64))


def test_linearity_and_scale_doubling():
    K, N, bits = 128, 64, 4
    L = gi.make_layer(K, N, bits, 32, desc_act=True, seed=5)
    rng = np.random.default_rng(3)
    x1 = gi.to_f16_bits(rng.integers(-8, 8, size=(2, K)))
    x2 = gi.to_f16_bits(rng.integers(-8, 8, size=(2, K)))
    xs = gi.to_f16_bits(o.decode_float_bits(x1, "f16") + o.decode_float_bits(x2, "f16"))   # exact
    f = lambda x, sc: o.gemm(x, "f16", L.qweight, L.qzeros, sc, "f16", L.g_idx, bits)
    y1, y2, ys = f(x1, L.scales), f(x2, L.scales), f(xs, L.scales)
    assert np.allclose(ys, y1 + y2, rtol=0, atol=1e-12 * np.abs(ys).max())
    s2 = gi.to_f16_bits(2 * o.decode_float_bits(L.scales, "f16"))
    assert np.array_equal(f(x1, s2), 2 * y1)


# ---- float formats and the comparison helper ---------------------------------------------------

def test_decode_float_bits():
    assert o.decode_float_bits(np.array([0x3C00, 0xC000, 0x7BFF], dtype=np.uint16), "f16").tolist() == [1.0, -2.0, 65504.0]
    assert o.decode_float_bits(np.array([0x3F80, 0x4049, 0xC2F7], dtype=np.uint16), "bf16").tolist() == [1.0, 3.140625, -123.5]


def test_bf16_rounding_against_brute_force_neighbours():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000),
                        [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 0.0, 3e38, 1e-40]])
    got = o.round_to_dtype_bits(v, "bf16")
    for val, g in zip(v, got):
        f32 = np.float32(val).view(np.uint32)
        cands = {int(f32 >> 16) + d for d in (-1, 0, 1, 2)}
        best = None
        for c in sorted(cands):
            if c & 0x7F80 == 0x7F80:
                continue
            cv = float(o.decode_float_bits(np.array([c], dtype=np.uint16), "bf16")[0])
            err = abs(Fraction(cv) - Fraction(float(val)))
            key = (err, c & 1)                       # ties go to the even pattern
            if best is None or key < best[0]:
                best = (key, c)
        assert int(g) == best[1], (val, hex(int(g)), hex(best[1]))
    assert o.round_to_dtype_bits(np.array([1 + 2.0 ** -8]), "bf16")[0] == 0x3F80


def test_compare_metrics():
    ref = np.array([[1.0, -2.0, 4.0, 0.5]])
    assert o.compare(o.round_to_dtype_bits(ref, "f16"), "f16", ref)["rel_l2"] == 0.0
    y = o.round_to_dtype_bits(ref * 1.0009765625, "f16")          # each value off by one part in 1024
    m = o.compare(y, "f16", ref)
    assert abs(m["rel_l2"] - 2.0 ** -10) < 1e-12 and abs(m["max_abs"] - 4.0 * 2.0 ** -10) < 1e-12


# ---- AWQ GEMM checkpoints (a second packing of the same W) ---------------------------------------

def test_awq_words_unpack_to_stated_codes():
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "awq_words.json")))
    for case in g["cases"]:
        w = np.array([[int(case["word_hex"], 16)]], dtype=np.uint64)
        assert o.unpack_awq(o.to_i32(w)).tolist() == [case["codes"]], case
        assert o.to_u32(o.pack_awq(np.array([case["codes"]]))).tolist() == [[int(case["word_hex"], 16)]]


def test_awq_single_hot_and_round_trip():
    for col in range(16):
        for v in (1, 7, 15):
            c = np.zeros((1, 16), dtype=np.uint8)
            c[0, col] = v
            w = o.to_u32(o.pack_awq(c))
            assert np.count_nonzero(w) == 1 and w[0, col // 8] == v << int(4 * o.AWQ_ORDER.index(col % 8))
    rng = np.random.default_rng(2)
    words = rng.integers(0, 2 ** 32, size=(5, 6), dtype=np.uint64)
    assert np.array_equal(o.to_u32(o.pack_awq(o.unpack_awq(o.to_i32(words)))), words.astype(np.uint32))


def test_awq_dequant_matches_exact_rationals_and_zero_is_representable():
    rng = np.random.default_rng(3)
    K, N, gs = 64, 16, 32
    codes = rng.integers(0, 16, size=(K, N))
    zeros = rng.integers(0, 16, size=(K // gs, N))
    zeros[0, :4] = 0                                            # AWQ stores zeros as they are
    scales = gi.to_f16_bits(rng.uniform(0.005, 0.02, size=(K // gs, N)))
    W = o.dequant_awq(o.pack_awq(codes), o.pack_awq(zeros), scales, "f16", gs)
    s = o.decode_float_bits(scales, "f16")
    for n in range(N):
        for k in range(0, K, 3):
            g = k // gs
            assert Fraction(float(W[n, k])) == (int(codes[k, n]) - int(zeros[g, n])) * Fraction(float(s[g, n]))
    assert np.array_equal(W[:4, :gs], (codes[:gs, :4] * s[0, :4]).T)


def test_awq_layer_equals_the_gptq_layer_of_the_same_codes():
    """Logical codes and zeros (1..15) packed both ways give the same W and y."""
    rng = np.random.default_rng(4)
    K, N, gs = 256, 32, 64
    codes = rng.integers(0, 16, size=(K, N))
    zeros = rng.integers(1, 16, size=(K // gs, N))
    scales = gi.to_f16_bits(rng.uniform(0.005, 0.02, size=(K // gs, N)))
    g_idx = (np.arange(K) // gs).astype(np.int32)
    Wa = o.dequant_awq(o.pack_awq(codes), o.pack_awq(zeros), scales, "f16", gs)
    Wg = o.dequant(o.pack_codes(codes, 4), o.pack_zeros(zeros, 4), scales, "f16", g_idx, 4)
    assert np.array_equal(Wa, Wg)
    x = gi.make_x(3, K, "bf16", seed=5)
    ya = o.gemm_awq(x, "bf16", o.pack_awq(codes), o.pack_awq(zeros), scales, "f16", gs)
    yg = o.gemm(x, "bf16", o.pack_codes(codes, 4), o.pack_zeros(zeros, 4), scales, "f16", g_idx, 4)
    assert np.allclose(ya, yg, rtol=1e-13, atol=1e-13)


# ---- GPTQ_P planar packing and GPTQ v2 zeros ------------------------------------------------------

def test_planar_words_unpack_to_stated_codes():
    """Hand-derived words ("Kernel Backends Reference", section "Planar packing")."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "planar_words.json")))
    for case in g["cases"]:
        bits = case["bits"]
        words = np.array([[int(h, 16)] for h in case["words_hex"]], dtype=np.uint32)
        assert o.planar_unpack_rows(o.to_i32(words), bits)[:, 0].tolist() == case["codes"], case["why"]
        assert o.to_u32(o.planar_pack_rows(np.array(case["codes"])[:, None], bits)).ravel().tolist() == \
            [int(h, 16) for h in case["words_hex"]], case["why"]
        # the same rule along the output dimension (qzeros)
        assert o.planar_unpack_cols(o.to_i32(words.T), bits)[0].tolist() == case["codes"]


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_single_plane_widths_are_continuous_packing(bits):
    """The page states that single-plane 2/4/8-bit layouts are bit-identical to continuous ones."""
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(96, 5))
    assert np.array_equal(o.planar_pack_rows(codes, bits), o.pack_codes(codes, bits))
    words = rng.integers(0, 2 ** 32, size=(3 * bits, 4), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(o.planar_unpack_rows(o.to_i32(words), bits), o.unpack_codes(o.to_i32(words), bits))


def test_planar_3bit_differs_from_continuous_3bit():
    """...and that planar 3-bit is not the continuous cross-word 3-bit layout."""
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 8, size=(64, 3))
    assert not np.array_equal(o.planar_pack_rows(codes, 3), o.pack_codes(codes, 3))
    assert np.array_equal(o.planar_unpack_rows(o.planar_pack_rows(codes, 3), 3), codes)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_planar_single_hot_and_round_trip(bits):
    """Each bit of each code lands in exactly one bit of one word of its own 32-code block, its
    plane's words come in low-to-high order, and every word pattern is a valid encoding."""
    lows = np.cumsum((0,) + o.PLANES[bits])               # first code bit of each plane
    for j in range(32):
        for b in range(bits):
            c = np.zeros((64, 1), dtype=np.int64)
            c[32 + j, 0] = 1 << b
            w = o.to_u32(o.planar_pack_rows(c, bits))[:, 0]
            assert np.count_nonzero(w) == 1 and bin(int(w.max())).count("1") == 1
            row = int(np.nonzero(w)[0][0])
            p = int(np.searchsorted(lows, b, side="right") - 1)
            wp = o.PLANES[bits][p]
            assert row == bits + lows[p] + j // (32 // wp)        # second block, plane p's rows
            assert int(w[row]) == 1 << (wp * (j % (32 // wp)) + b - lows[p])
    rng = np.random.default_rng(100 + bits)
    words = rng.integers(0, 2 ** 32, size=(2 * bits, 6), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(o.to_u32(o.planar_pack_rows(o.planar_unpack_rows(o.to_i32(words), bits), bits)), words)


@pytest.mark.parametrize("bits", [3, 5, 6, 7])
def test_planar_dequant_matches_exact_rationals(bits):
    """GPTQ_P W = (code - (stored + 1)) * scale, brute force in exact rationals, act-order g_idx."""
    rng = np.random.default_rng(20 + bits)
    K, N, gs = 64, 32, 32
    codes = rng.integers(0, 1 << bits, size=(K, N))
    stored = rng.integers(0, 1 << bits, size=(K // gs, N))
    g_idx = (rng.permutation(K) // gs).astype(np.int32)
    scales = gi.to_bf16_bits(rng.uniform(0.005, 0.02, size=(K // gs, N)))
    W = o.dequant_fmt("gptq_p", o.planar_pack_rows(codes, bits), o.planar_pack_cols(stored, bits), scales, "bf16",
                      g_idx, bits)
    s = o.decode_float_bits(scales, "bf16")
    for n in range(N):
        for k in range(K):
            g = int(g_idx[k])
            assert Fraction(float(W[n, k])) == (int(codes[k, n]) - int(stored[g, n]) - 1) * Fraction(float(s[g, n]))
    x = gi.make_x(2, K, "f16", seed=bits)
    y = o.gemm_fmt("gptq_p", x, "f16", o.planar_pack_rows(codes, bits), o.planar_pack_cols(stored, bits), scales,
                   "bf16", g_idx, bits)
    xf = o.decode_float_bits(x, "f16")
    for m in range(2):
        for n in range(0, N, 7):
            exact = sum(Fraction(float(xf[m, k])) * Fraction(float(W[n, k])) for k in range(K))
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 60)


def test_planar_layer_of_a_single_plane_width_equals_the_gptq_layer():
    L = gi.make_layer(128, 64, 4, 32, desc_act=True, seed=31)
    assert np.array_equal(o.dequant_fmt("gptq_p", L.qweight, L.qzeros, L.scales, "f16", L.g_idx, 4),
                          o.dequant(L.qweight, L.qzeros, L.scales, "f16", L.g_idx, 4))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_v2_zeros_are_stored_as_they_are(bits):
    """A v2 layer storing z equals the v1 layer storing z - 1 (the same logical zero), and a v2
    zero of 0 is representable: W = code * scale there."""
    rng = np.random.default_rng(40 + bits)
    K, N, gs = 96, 32, 32
    L = gi.make_layer(K, N, bits, gs, desc_act=True, seed=40 + bits)
    zeros = rng.integers(0, 1 << bits, size=(K // gs, N))
    zeros[0, :3] = 0
    W2 = o.dequant_fmt("gptq_v2", L.qweight, o.pack_along_cols(zeros, bits), L.scales, "f16", L.g_idx, bits)
    codes = o.unpack_codes(L.qweight, bits)
    s = o.decode_float_bits(L.scales, "f16")
    g = L.g_idx.astype(np.int64)
    assert np.array_equal(W2, ((codes - zeros[g]) * s[g]).T)
    ok = zeros[:, :] >= 1                                   # where v1 can express the same zero
    W1 = o.dequant(L.qweight, o.pack_along_cols(np.where(ok, zeros - 1, 0), bits), L.scales, "f16", L.g_idx, bits)
    cols = np.all(ok, axis=0)
    assert cols.sum() > 0 and np.array_equal(W1[cols], W2[cols])
    first = np.nonzero(g == 0)[0]
    assert np.array_equal(W2[:3][:, first], (codes[first][:, :3] * s[0, :3]).T)
