"""Pins of the GPTQ quantizer oracle (oracle.quant) against what the page and the mathematics fix:
it must reduce to round-to-nearest when the Hessian is a multiple of the identity, agree with the
sequential Optimal-Brain-Quantization elimination written from the explicit inverse Hessian (no
Cholesky, no lazy batching), not depend on the lazy block size, lower the layer's output error
below round-to-nearest's, and zero never-active inputs exactly.  The Hessian 2 X^T X / n and the
output-error objective are pinned by hand-worked values and exact rationals ("39. Quantized
checkpoints ...", section "GPTQ": the objective and H = 2 X^T X)."""
import numpy as np
import pytest

import oracle as o

q = o.quant


def correlated_inputs(S, K, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((K, K)) * 0.3 + np.eye(K)
    return (rng.standard_normal((S, K)) @ A).astype(np.float32)


def test_find_params_grid_contains_zero_and_the_range():
    a = np.array([[-1.0, 0.5, 2.0], [0.25, 0.5, 1.0], [0.0, 0.0, 0.0], [-3.0, -1.0, -2.0]], dtype=np.float32)
    s, z = q.find_params(a, 4)
    assert np.allclose(s, [3.0 / 15, 1.0 / 15, 1.0, 3.0 / 15]) and np.array_equal(z, [5, 0, 0, 15])
    for r in range(4):                                   # 0 is a grid point; the range fits the grid
        assert s[r] * (0 - z[r]) <= a[r].min() + 1e-6 or a[r].min() >= 0
        assert s[r] * (15 - z[r]) >= a[r].max() - s[r] / 2


@pytest.mark.parametrize("bits,gs", [(4, 32), (3, 64), (2, -1), (8, 32)])
def test_identity_hessian_is_round_to_nearest(bits, gs):
    rng = np.random.default_rng(bits)
    N, K = 24, 128
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    H = np.eye(K, dtype=np.float32) * np.float32(3.0)
    c, s, z, g = q.gptq_quantize(W, H, bits, gs)
    cr, sr, zr, gr = q.rtn_quantize(W, bits, gs)
    assert np.array_equal(c, cr) and np.array_equal(s, sr) and np.array_equal(z, zr) and np.array_equal(g, gr)


def test_diagonal_hessian_with_act_order_is_round_to_nearest_in_visiting_order():
    rng = np.random.default_rng(7)
    N, K, gs = 16, 128, 32
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    d = rng.permutation(K).astype(np.float32) + 1.0                 # distinct activations
    c, s, z, g = q.gptq_quantize(W, np.diag(d), 4, gs, act_order=True)
    order = np.argsort(-d)                                          # most active input first
    cr, sr, zr, _ = q.rtn_quantize(W[:, order], 4, gs)
    back = np.argsort(order)
    assert np.array_equal(c, cr[:, back]) and np.array_equal(s, sr) and np.array_equal(z, zr)
    assert np.array_equal(g, (np.arange(K) // gs)[back])
    assert np.array_equal(np.sort(g), np.arange(K) // gs)          # whole groups (r6)


def obq_sequential(W, H, bits, gs, damp=0.01):
    """Optimal Brain Quantization in the column order 0..K-1, float64: quantize column i, push its
    error through the current inverse Hessian, then eliminate i from it (no Cholesky, no blocks)."""
    W = np.array(W, dtype=np.float64)
    H = np.array(H, dtype=np.float64)
    K = W.shape[1]
    H = H + damp * np.diag(H).mean() * np.eye(K)
    Hinv = np.linalg.inv(H)
    top = 2 ** bits - 1
    codes = np.zeros(W.shape, dtype=np.int64)
    s = z = None
    for i in range(K):
        if i % gs == 0:
            blk = W[:, i:i + gs]
            lo, hi = np.minimum(blk.min(1), 0), np.maximum(blk.max(1), 0)
            s = (hi - lo) / top
            z = np.round(-lo / s)
        qi = np.clip(np.round(W[:, i] / s + z), 0, top)
        codes[:, i] = qi
        e = (W[:, i] - s * (qi - z)) / Hinv[i, i]
        W[:, i + 1:] -= np.outer(e, Hinv[i, i + 1:])
        Hinv = Hinv - np.outer(Hinv[:, i], Hinv[i, :]) / Hinv[i, i]
    return codes


@pytest.mark.parametrize("bits", [2, 4])
def test_matches_sequential_obq_from_the_explicit_inverse(bits):
    rng = np.random.default_rng(10 + bits)
    N, K, gs = 12, 64, 16
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    H = q.hessian(correlated_inputs(256, K, 20 + bits))
    c, _, _, _ = q.gptq_quantize(W, H, bits, gs, block=16)      # lazy blocks of 16 across 4 blocks
    ref = obq_sequential(W, H, bits, gs)
    assert np.array_equal(c.astype(np.int64), ref)


def test_lazy_block_size_does_not_change_the_result():
    rng = np.random.default_rng(5)
    N, K, gs = 20, 128, 16
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    H = q.hessian(correlated_inputs(256, K, 6))
    a = q.gptq_quantize(W, H, 4, gs, block=128)
    b = q.gptq_quantize(W, H, 4, gs, block=16)
    assert np.array_equal(a[0], b[0]) and np.allclose(a[1], b[1], rtol=1e-5) and np.array_equal(a[2], b[2])


@pytest.mark.parametrize("bits,act", [(2, False), (3, True), (4, False), (4, True)])
def test_output_error_below_round_to_nearest(bits, act):
    rng = np.random.default_rng(bits + 10 * act)
    N, K, S = 48, 192, 512
    X = correlated_inputs(S, K, 30 + bits)
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    c, s, z, g = q.gptq_quantize(W, q.hessian(X), bits, 64, act_order=act)
    assert c.max() <= 2 ** bits - 1 and z.min() >= 0 and z.max() <= 2 ** bits - 1 and s.min() > 0
    cr, sr, zr, gr = q.rtn_quantize(W, bits, 64)
    assert q.layer_loss(W, c, s, z, g, X) < 0.8 * q.layer_loss(W, cr, sr, zr, gr, X)


def test_never_active_inputs_quantize_to_exact_zero():
    rng = np.random.default_rng(8)
    N, K = 16, 96
    X = correlated_inputs(128, K, 9)
    X[:, [3, 50, 77]] = 0
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    c, s, z, g = q.gptq_quantize(W, q.hessian(X), 4, 32, act_order=True)
    deq = s[:, g] * (c.astype(np.float32) - z[:, g])
    assert np.all(deq[:, [3, 50, 77]] == 0)


def test_hessian_hand_computed_two_inputs():
    """H = 2 X^T X / n worked by hand: X = [[1, 0], [2, 1], [0, 3], [1, 1]] (n = 4) gives
    X^T X = [[6, 3], [3, 11]], so H = [[3, 1.5], [1.5, 5.5]] (a dropped factor 2 or a dropped 1/n
    gives another matrix)."""
    X = np.array([[1, 0], [2, 1], [0, 3], [1, 1]], dtype=np.float32)
    H = q.hessian(X)
    assert H.dtype == np.float32
    assert np.array_equal(H, np.array([[3.0, 1.5], [1.5, 5.5]], dtype=np.float32))


def test_hessian_exact_rationals():
    """Every entry equals the exact rational sum over rows of 2 x_s,i x_s,j / n, rounded once to
    float32 (inputs on a dyadic grid, so the rational is computed without error)."""
    from fractions import Fraction
    rng = np.random.default_rng(11)
    n, K = 7, 5
    X = (rng.integers(-64, 65, size=(n, K)) / 16.0).astype(np.float32)
    H = q.hessian(X)
    for i in range(K):
        for j in range(K):
            exact = sum(Fraction(float(X[s, i])) * Fraction(float(X[s, j])) for s in range(n)) * 2 / n
            assert H[i, j] == np.float32(float(exact)), (i, j)
    assert np.array_equal(H, H.T)


def test_layer_loss_hand_computed():
    """||X Wq^T - X W^T||^2 worked by hand.  W = [[1, -2], [0.5, 0]]; the codes, scales and zeros
    give Wq = [[1.5, -2], [0.5, 0.25]] (one group: scale 0.25, zeros 8 and 2), so Wq - W =
    [[0.5, 0], [0, 0.25]]; with X = [[2, 1], [0, 3]], X (Wq - W)^T = [[1, 0.25], [0, 0.75]] and the
    loss is 1 + 0.0625 + 0 + 0.5625 = 1.625."""
    W = np.array([[1.0, -2.0], [0.5, 0.0]], dtype=np.float32)
    codes = np.array([[14, 0], [4, 3]], dtype=np.uint8)
    scales = np.array([[0.25], [0.25]], dtype=np.float32)
    zeros = np.array([[8], [2]], dtype=np.int32)
    g_idx = np.array([0, 0], dtype=np.int32)
    X = np.array([[2.0, 1.0], [0.0, 3.0]])
    assert q.layer_loss(W, codes, scales, zeros, g_idx, X) == 1.625
    # and it is zero exactly when the quantized weights equal the weights
    assert q.layer_loss(scales[:, [0, 0]] * (codes.astype(np.float32) - zeros[:, [0, 0]]), codes, scales, zeros,
                        g_idx, X) == 0.0


def test_layer_loss_uses_g_idx():
    """With act-order groups the loss reads each input's own group: swapping g_idx changes it."""
    W = np.zeros((1, 2), dtype=np.float32)
    codes = np.array([[1, 1]], dtype=np.uint8)
    scales = np.array([[1.0, 2.0]], dtype=np.float32)
    zeros = np.array([[0, 0]], dtype=np.int32)
    X = np.array([[1.0, 0.0]])
    assert q.layer_loss(W, codes, scales, zeros, np.array([0, 1], dtype=np.int32), X) == 1.0
    assert q.layer_loss(W, codes, scales, zeros, np.array([1, 0], dtype=np.int32), X) == 4.0
