"""Plain CPU oracle for the GPTQ quantizer, the step that produces a layer's codes, scales and zeros.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke entry and the bench's
CPU baseline may import it.  numpy in float32 wherever the method works on float32 copies of the
weight and the Hessian, so that every rounding decision that fixes a code is taken in the same
precision as the GPU quantizer; the Hessian itself is summed in float64 and rounded once.

Written from the statements of "39. Quantized checkpoints: GPTQ, AWQ, FP8, FP4 and trellis codes",
section "GPTQ":
  * objective: the squared output error ||X Wq^T - X W^T||^2 on calibration inputs X, a quadratic
    in each weight row with one Hessian shared by all rows, H = 2 X^T X (the quantizer is handed
    H averaged over the n calibration rows, 2 X^T X / n);
  * columns are quantized one after another; once column i is fixed, its rounding error, divided
    by the i-th diagonal entry of the inverse Hessian of the columns still free, is subtracted from
    every later column j in proportion to entry (i, j) of that inverse (the error-feedback equation);
  * that shrinking inverse is never formed: its rows are read off the upper Cholesky factor U of
    the inverse of the damped Hessian (damping adds a fraction of the mean diagonal to the
    diagonal).  Row i of U is row i of the free-column inverse divided by the square root of its
    diagonal entry, so the scaled error (w_i - q_i) / U_ii times U_ij is exactly the update the
    equation asks for;
  * lazy batches: within a batch of 128 columns every error is applied to the batch's later columns
    at once; the columns after the batch receive all of the batch's errors in one matrix product
    when the batch is done;
  * an input that is never active (H_ii = 0) carries no information: its diagonal becomes 1 and its
    weights 0;
  * act-order visits the inputs from the largest H_ii down; groups are runs of group_size columns in
    visiting order, and g_idx gives each original input its group;
  * a group's grid is taken from the corrected weights at the moment the sweep reaches the group's
    first column.

Readings where the page leaves a step open (listed with the others in the design notes):
  * the grid ("find_params" is named, not defined): asymmetric min-max over a row's current group
    values, widened to contain 0 so that 0 is exact: lo = min(0, min w), hi = max(0, max w),
    scale = (hi - lo) / (2^bits - 1), zero = round(-lo / scale) (round half to even); a group of
    zeros takes scale 1, zero 0;
  * the quantizer q = scale * (clamp(round(w / scale + zero), 0, 2^bits - 1) - zero);
  * "corrected weights" under lazy batches: when a group's window reaches past the current batch,
    the columns past it carry the corrections of the earlier batches only (their share of the
    current batch arrives with the batch's product).  With group sizes that divide the batch or
    are multiples of it the window is fully corrected either way;
  * the inverse factor follows the three steps the page names: Cholesky factor of the damped
    Hessian, the inverse rebuilt from that factor, the upper Cholesky factor of the inverse.
"""
from __future__ import annotations

import numpy as np

__all__ = ["hessian", "find_params", "gptq_quantize", "rtn_quantize", "layer_loss"]

F32 = np.float32


def hessian(x) -> np.ndarray:
    """H = 2 X^T X / n of calibration inputs X [n, K] (the Hessian of the squared output error,
    averaged over the n rows): float64 products and sums, rounded once to float32."""
    X = np.asarray(x, dtype=np.float64)
    n = X.shape[0]
    return ((X.T @ X) * (2.0 / n)).astype(F32)


def find_params(values, bits: int):
    """Grid of each row of `values` [rows, cols] (the reading in the module docstring): returns
    (scale, zero), float32 [rows]."""
    v = np.asarray(values, dtype=F32)
    qmax = F32(2 ** bits - 1)
    low = np.minimum(v.min(axis=1), F32(0))
    high = np.maximum(v.max(axis=1), F32(0))
    empty = high == low
    step = np.where(empty, F32(1), (high - low) / qmax).astype(F32)
    offset = np.where(empty, F32(0), np.round(-low / step)).astype(F32)
    return step, offset


def _visiting_order(diag, act_order: bool) -> np.ndarray:
    """Columns in the order the sweep visits them: the most active input first (stable among equal
    diagonals) with act-order, else input order."""
    if not act_order:
        return np.arange(diag.shape[0])
    return np.argsort(-diag, kind="stable")


def _inverse_factor(Hv) -> np.ndarray:
    """Upper Cholesky factor U of Hv^-1 (Hv^-1 = U^T U), float32, through the Cholesky factor of Hv:
    Hv = C C^T, Hv^-1 = C^-T C^-1, then the upper factor of that."""
    C = np.linalg.cholesky(Hv)                                   # lower, float32 LAPACK
    C_inv = np.linalg.inv(C).astype(F32)
    Hv_inv = (C_inv.T @ C_inv).astype(F32)
    return np.linalg.cholesky(Hv_inv).T.astype(F32)


def gptq_quantize(weight, H, bits: int = 4, group_size: int = 128, act_order: bool = False,
                  damp: float = 0.01, block: int = 128):
    """GPTQ of weight [N, K] (rows are outputs) against H [K, K].  Returns codes uint8 [N, K] in the
    original input order, scales float32 [N, G], zeros int32 [N, G] (logical zeros, 0..2^bits - 1)
    and g_idx int32 [K].  group_size -1 means one group over all inputs; `block` is the lazy batch."""
    Wv = np.array(weight, dtype=F32)            # becomes the weights in visiting order, corrected
    Hv = np.array(H, dtype=F32)
    n_out, n_in = Wv.shape
    width = n_in if group_size == -1 else group_size
    qmax = F32(2 ** bits - 1)

    silent = np.flatnonzero(np.diag(Hv) == 0)
    Hv[silent, silent] = F32(1)
    Wv[:, silent] = F32(0)

    order = _visiting_order(np.diag(Hv), act_order)
    Wv = Wv[:, order]
    Hv = Hv[np.ix_(order, order)]
    Hv[np.diag_indices(n_in)] += F32(damp) * np.diag(Hv).mean(dtype=F32)
    U = _inverse_factor(Hv)

    n_groups = -(-n_in // width)
    codes_v = np.zeros((n_out, n_in), dtype=F32)
    scale = np.zeros((n_out, n_groups), dtype=F32)
    zero = np.zeros((n_out, n_groups), dtype=F32)
    for first in range(0, n_in, block):
        last = min(first + block, n_in)           # this batch is columns [first, last)
        scaled_err = np.zeros((n_out, last - first), dtype=F32)
        for c in range(first, last):
            g = c // width
            if c == g * width:
                scale[:, g], zero[:, g] = find_params(Wv[:, c:c + width], bits)
            s, z = scale[:, g], zero[:, g]
            code = np.clip(np.round(Wv[:, c] / s + z), F32(0), qmax).astype(F32)
            codes_v[:, c] = code
            e = ((Wv[:, c] - s * (code - z)) / U[c, c]).astype(F32)
            scaled_err[:, c - first] = e
            Wv[:, c + 1:last] -= np.outer(e, U[c, c + 1:last]).astype(F32)
        if last < n_in:
            Wv[:, last:] -= (scaled_err @ U[first:last, last:]).astype(F32)

    position = np.empty(n_in, dtype=np.int64)     # visiting position of each original input
    position[order] = np.arange(n_in)
    g_idx = (position // width).astype(np.int32)
    return codes_v[:, position].astype(np.uint8), scale, zero.astype(np.int32), g_idx


def rtn_quantize(weight, bits: int = 4, group_size: int = 128):
    """Round-to-nearest with the same per-group grid over the ORIGINAL weights (no error feedback):
    what GPTQ must reduce to when H is a multiple of the identity."""
    W = np.asarray(weight, dtype=F32)
    K = W.shape[1]
    gs = K if group_size == -1 else group_size
    qmax = F32(2 ** bits - 1)
    G = -(-K // gs)
    codes = np.zeros(W.shape, dtype=np.uint8)
    scales = np.zeros((W.shape[0], G), dtype=F32)
    zeros = np.zeros((W.shape[0], G), dtype=F32)
    for g in range(G):
        blk = W[:, g * gs:(g + 1) * gs]
        scales[:, g], zeros[:, g] = find_params(blk, bits)
        codes[:, g * gs:(g + 1) * gs] = np.clip(np.round(blk / scales[:, g:g + 1] + zeros[:, g:g + 1]), 0, qmax)
    return codes, scales, zeros.astype(np.int32), (np.arange(K) // gs).astype(np.int32)


def layer_loss(weight, codes, scales, zeros, g_idx, X) -> float:
    """||X Wq^T - X W^T||^2 in float64 with Wq[n, k] = scale[n, g] (code[n, k] - zero[n, g]),
    g = g_idx[k]: the objective the quantizer minimises."""
    W = np.asarray(weight, dtype=np.float64)
    g = np.asarray(g_idx, dtype=np.int64)
    Wq = np.asarray(scales, dtype=np.float64)[:, g] * (codes.astype(np.float64) - np.asarray(zeros, np.float64)[:, g])
    D = np.asarray(X, dtype=np.float64) @ (Wq - W).T
    return float((D * D).sum())
