"""Plain CPU oracle for the GPTQ quantizer: the step that produces a layer's codes, scales and zeros.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy, in float32 where the page computes in
float32 (it takes `.float()` copies of the weight and the Hessian), so that every rounding decision
that fixes a code is taken in the same precision as the GPU quantizer; the Hessian itself is
accumulated in float64 and rounded once.

Source: "39. Quantized checkpoints: GPTQ, AWQ, FP8, FP4 and trellis codes", section "GPTQ":
  * the objective min ||X W^T - X What^T||^2, the shared per-row Hessian H = 2 X^T X (the
    quantizer takes H = 2 X^T X / n);
  * columns are quantized one at a time and each error e = (w_i - quant(w_i)) / [H^-1]_ii is
    pushed onto the later columns through row i of the inverse Hessian;
  * the inverse Hessian comes from a Cholesky factorization of the damped H (damp times the mean
    diagonal added to the diagonal), as the upper Cholesky factor of H^-1;
  * lazy batch updates: inside a block of 128 columns each error updates the block, the columns
    after the block are updated with one matrix product when the block is done;
  * inputs that are never active (H_ii = 0) get H_ii = 1 and zero weights;
  * act-order visits columns from the largest H_ii down; groups are consecutive in the visiting
    order and g_idx maps each original column to its group;
  * a group's range is taken from the CURRENT (already corrected) weights when the loop enters it,
    over the next group_size columns.

Readings where the page is silent:
  * the per-group parameters ("find_params" is named, not printed): an asymmetric min-max grid
    over each row's group values, widened to contain 0 so that 0 is exact (lo = min(0, min w),
    hi = max(0, max w)); scale = (hi - lo) / (2^bits - 1), zero = round(-lo / scale); a group that
    is all zeros takes scale 1, zero 0.  float32 arithmetic, round half to even.
  * quant(w) = scale * (clamp(round(w / scale + zero), 0, 2^bits - 1) - zero), as printed.
"""
from __future__ import annotations

import numpy as np

__all__ = ["hessian", "find_params", "gptq_quantize", "rtn_quantize", "layer_loss"]


def hessian(x) -> np.ndarray:
    """H = 2 X^T X / n for calibration inputs X [n, K] (float values), float64 product rounded once
    to float32 (the quantizer's precision)."""
    X = np.asarray(x, dtype=np.float64)
    return (2.0 * (X.T @ X) / X.shape[0]).astype(np.float32)


def find_params(ahead, bits: int):
    """Per-row scale and zero of a group from its current values `ahead` [rows, cols] (the reading
    in the module docstring).  float32."""
    a = np.asarray(ahead, dtype=np.float32)
    top = np.float32(2 ** bits - 1)
    lo = np.minimum(a.min(axis=1), np.float32(0))
    hi = np.maximum(a.max(axis=1), np.float32(0))
    flat = hi == lo
    span = np.where(flat, np.float32(1), hi - lo).astype(np.float32)
    scale = np.where(flat, np.float32(1), span / top).astype(np.float32)
    zero = np.where(flat, np.float32(0), np.round(-lo / scale)).astype(np.float32)
    return scale, zero


def gptq_quantize(weight, H, bits: int = 4, group_size: int = 128, act_order: bool = False,
                  damp: float = 0.01, block: int = 128):
    """weight [N, K] (float), H [K, K] -> (codes uint8 [N, K] in original column order,
    scales float32 [N, G], zeros int32 [N, G], g_idx int32 [K]), following the page's steps in
    order.  group_size -1 means one group of all K columns."""
    W = np.array(weight, dtype=np.float32)
    H = np.array(H, dtype=np.float32)
    K = W.shape[1]
    gs = K if group_size == -1 else group_size
    top = np.float32(2 ** bits - 1)
    dead = np.diag(H) == 0                      # never-active inputs: their weights do not matter
    H[dead, dead] = 1
    W[:, dead] = 0
    perm = np.argsort(-np.diag(H), kind="stable") if act_order else np.arange(K)
    W = W[:, perm]
    H = H[perm][:, perm]
    H = H + np.float32(damp) * np.diag(H).mean(dtype=np.float32) * np.eye(K, dtype=np.float32)
    L = np.linalg.cholesky(H)                                   # H = L L^T
    Hi = np.linalg.inv(L @ L.T).astype(np.float32)             # cholesky_inverse: (L L^T)^-1
    Hi = (Hi + Hi.T) / np.float32(2)                            # (inv returns a full matrix)
    U = np.linalg.cholesky(Hi).T.astype(np.float32)            # upper factor: Hi = U^T U
    G = -(-K // gs)
    codes = np.zeros(W.shape, dtype=np.float32)
    scales = np.zeros((W.shape[0], G), dtype=np.float32)
    zeros = np.zeros((W.shape[0], G), dtype=np.float32)
    for i1 in range(0, K, block):
        i2 = min(i1 + block, K)
        W1 = W[:, i1:i2].copy()
        Err = np.zeros((W.shape[0], i2 - i1), dtype=np.float32)
        U1 = U[i1:i2, i1:i2]
        for i in range(i2 - i1):
            col = i1 + i
            g = col // gs
            if col % gs == 0:                  # a new group: its range from the corrected weights
                ahead = np.concatenate((W1[:, i:], W[:, i2:]), axis=1)[:, :gs]
                scales[:, g], zeros[:, g] = find_params(ahead, bits)
            q = np.clip(np.round(W1[:, i] / scales[:, g] + zeros[:, g]), 0, top).astype(np.float32)
            codes[:, col] = q
            err = ((W1[:, i] - scales[:, g] * (q - zeros[:, g])) / U1[i, i]).astype(np.float32)
            W1[:, i:] -= err[:, None] * U1[i, i:][None, :]      # correct the rest of the block
            Err[:, i] = err
        W[:, i2:] -= Err @ U[i1:i2, i2:]                        # and everything after it
    inverse = np.argsort(perm, kind="stable")
    g_idx = (np.arange(K) // gs)[inverse].astype(np.int32)
    return codes[:, inverse].astype(np.uint8), scales, zeros.astype(np.int32), g_idx


def rtn_quantize(weight, bits: int = 4, group_size: int = 128):
    """Round-to-nearest with the same per-group grid over the ORIGINAL weights (no error feedback):
    what GPTQ must reduce to when H is a multiple of the identity."""
    W = np.asarray(weight, dtype=np.float32)
    K = W.shape[1]
    gs = K if group_size == -1 else group_size
    top = np.float32(2 ** bits - 1)
    G = -(-K // gs)
    codes = np.zeros(W.shape, dtype=np.uint8)
    scales = np.zeros((W.shape[0], G), dtype=np.float32)
    zeros = np.zeros((W.shape[0], G), dtype=np.float32)
    for g in range(G):
        blk = W[:, g * gs:(g + 1) * gs]
        scales[:, g], zeros[:, g] = find_params(blk, bits)
        codes[:, g * gs:(g + 1) * gs] = np.clip(np.round(blk / scales[:, g:g + 1] + zeros[:, g:g + 1]), 0, top)
    return codes, scales, zeros.astype(np.int32), (np.arange(K) // gs).astype(np.int32)


def layer_loss(weight, codes, scales, zeros, g_idx, X) -> float:
    """||X What^T - X W^T||^2 in float64 with What[n, k] = scale[n, g] (code[n, k] - zero[n, g]),
    g = g_idx[k] (the objective the page states)."""
    W = np.asarray(weight, dtype=np.float64)
    g = np.asarray(g_idx, dtype=np.int64)
    Wh = np.asarray(scales, dtype=np.float64)[:, g] * (codes.astype(np.float64) - np.asarray(zeros, np.float64)[:, g])
    D = np.asarray(X, dtype=np.float64) @ (Wh - W).T
    return float((D * D).sum())
