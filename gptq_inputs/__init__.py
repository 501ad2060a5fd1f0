"""Seeded synthetic inputs for the GPTQ linear layer (shared by tests and the benchmark).

This module holds NO arithmetic of the method: it only draws random numbers with the
shapes and value distributions of the workloads below and rounds real-valued draws to
the storage dtype.  Packed words are drawn directly as uniform random 32-bit words: every
bit pattern is a valid word, and uniform words make every b-bit code (and every stored
zero) uniform over [0, 2**b - 1], which is the distribution the workloads ask for
("codes uniform over [0, 2**b - 1]; zeros uniform over the same range, stored minus one").

Floating-point arrays are returned as raw uint16 bit patterns tagged "f16" / "bf16"
(or float32 values tagged "f32") so that neither consumer has to trust the other's
float conversion.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Layer", "AwqLayer", "make_layer", "make_awq_layer", "make_x", "make_bias", "make_weight", "make_calib",
           "to_f16_bits",
           "to_bf16_bits", "WORKLOADS", "seed_for"]


def to_f16_bits(v) -> np.ndarray:
    """float64 draws -> fp16 bit patterns (numpy's float64->float16 cast rounds to nearest even)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_bf16_bits(v) -> np.ndarray:
    """float64 draws -> bf16 bit patterns: round to float32, then round-to-nearest-even on the
    top 16 bits.  (The rounded arrays ARE the inputs; the route of the rounding is immaterial.)"""
    u = np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def _round(v, dtype):
    if dtype == "f16":
        return to_f16_bits(v)
    if dtype == "bf16":
        return to_bf16_bits(v)
    if dtype == "f32":
        return np.asarray(v, dtype=np.float32)
    raise ValueError(dtype)


@dataclasses.dataclass
class Layer:
    K: int
    N: int
    bits: int
    group_size: int
    desc_act: bool
    qweight: np.ndarray      # int32 [K*bits/32, N]
    qzeros: np.ndarray       # int32 [G, N*bits/32]
    scales: np.ndarray       # uint16 bits (f16/bf16) or float32, [G, N]
    scales_dtype: str
    g_idx: np.ndarray        # int32 [K]

    @property
    def G(self) -> int:
        return self.scales.shape[0]


def make_layer(K, N, bits, group_size, desc_act=False, scales_dtype="f16", seed=0,
               scale_lo=0.005, scale_hi=0.02) -> Layer:
    """Draw one checkpoint layer.

    Draw order: qweight words, qzeros words, scales ~ U[scale_lo, scale_hi) (rounded to
    scales_dtype), then for desc_act a permutation p of range(K) with g_idx = p // gs;
    otherwise g_idx = k // gs.  group_size = -1 gives one group (g_idx = 0).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    gs = K if group_size == -1 else group_size
    G = -(-K // gs)
    qweight = rng.integers(0, 2 ** 32, size=(K * bits // 32, N), dtype=np.uint64).astype(np.uint32).view(np.int32)
    qzeros = rng.integers(0, 2 ** 32, size=(G, N * bits // 32), dtype=np.uint64).astype(np.uint32).view(np.int32)
    scales = _round(rng.uniform(scale_lo, scale_hi, size=(G, N)), scales_dtype)
    if desc_act:
        g_idx = (rng.permutation(K) // gs).astype(np.int32)
    else:
        g_idx = (np.arange(K) // gs).astype(np.int32)
    return Layer(K, N, bits, group_size, bool(desc_act), qweight, qzeros, scales, scales_dtype, g_idx)


@dataclasses.dataclass
class AwqLayer:
    K: int
    N: int
    group_size: int
    qweight: np.ndarray      # int32 [K, N/8]  (AutoAWQ GEMM: eight 4-bit fields along the outputs)
    qzeros: np.ndarray       # int32 [G, N/8]
    scales: np.ndarray       # uint16 bits (f16/bf16) or float32, [G, N]
    scales_dtype: str
    bits: int = 4

    @property
    def G(self) -> int:
        return self.scales.shape[0]


def make_awq_layer(K, N, group_size, scales_dtype="f16", seed=0, scale_lo=0.005, scale_hi=0.02) -> AwqLayer:
    """Draw one 4-bit AutoAWQ GEMM layer: uniform qweight words [K, N/8], uniform qzeros words
    [G, N/8] (so every code and zero is uniform over [0, 15] whatever the field order), then
    scales ~ U[scale_lo, scale_hi) rounded to scales_dtype."""
    rng = np.random.Generator(np.random.PCG64(seed))
    gs = K if group_size == -1 else group_size
    G = -(-K // gs)
    qweight = rng.integers(0, 2 ** 32, size=(K, N // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
    qzeros = rng.integers(0, 2 ** 32, size=(G, N // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
    scales = _round(rng.uniform(scale_lo, scale_hi, size=(G, N)), scales_dtype)
    return AwqLayer(K, N, group_size, qweight, qzeros, scales, scales_dtype)


def make_weight(N, K, seed=0, std=0.02) -> np.ndarray:
    """A float layer weight [N, K] ~ N(0, std^2), float32 (the quantizer's input)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((N, K)) * std).astype(np.float32)


def make_calib(S, K, dtype="bf16", seed=0) -> np.ndarray:
    """Calibration activations [S, K] with correlated inputs: z A with z ~ N(0, 1) and
    A = I + N(0, 0.25 / K) entries, rounded to the activation dtype (bit patterns)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    A = rng.standard_normal((K, K)) * (0.5 / np.sqrt(K)) + np.eye(K)
    return _round(rng.standard_normal((S, K)) @ A, dtype)


def make_x(M, K, dtype="f16", seed=0) -> np.ndarray:
    """Activations x[M, K] ~ N(0, 1), rounded to the activation dtype (bit patterns)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _round(rng.standard_normal(size=(M, K)), dtype)


def make_bias(N, dtype="f16", seed=0) -> np.ndarray:
    """A layer's bias[N] ~ N(0, 1), rounded to the scales' dtype (bit patterns, or float32)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _round(rng.standard_normal(size=N), dtype)


def seed_for(workload: int, variant: int = 0) -> int:
    return 20261202 + 1000 * workload + 10 * variant


# The five workloads (shapes and distributions of the layers the pages discuss).  Each entry:
# name, K, N, list of M, bits list, group sizes, desc_act, scales dtype, activation dtype.
WORKLOADS = [
    dict(name="tiny_256x256", K=256, N=256, Ms=[1], bits=[4], group_sizes=[128], desc_act=False,
         scales_dtype="f16", x_dtype="f16"),
    dict(name="llama3_8b_up_proj", K=4096, N=14336, Ms=[1, 4, 16], bits=[4], group_sizes=[128],
         desc_act=False, scales_dtype="f16", x_dtype="f16"),
    dict(name="llama3_70b_gate_proj", K=8192, N=28672, Ms=[1, 8, 16], bits=[4], group_sizes=[128],
         desc_act=False, scales_dtype="f16", x_dtype="bf16"),
    dict(name="act_order_width_sweep", K=8192, N=8192, Ms=[1, 32], bits=[2, 3, 4, 8],
         group_sizes=[128, -1], desc_act=True, scales_dtype="f16", x_dtype="f16"),
    dict(name="prefill_4096x8192x28672", K=8192, N=28672, Ms=[4096], bits=[4], group_sizes=[128],
         desc_act=False, scales_dtype="bf16", x_dtype="bf16"),
]
