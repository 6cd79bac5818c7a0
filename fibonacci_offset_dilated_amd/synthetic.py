"""Seeded synthetic inputs shared by the HIP path, its tests, the bench and the CPU oracle runs.

This module holds none of the attention method's arithmetic. It draws random numbers, casts
fp32 draws to bf16 (round to nearest even, done on the bit pattern), and states the seed
recipe. Both sides of every parity check receive the very same arrays from here.

Input recipe (the trained models and text corpora the pages evaluate on are not available,
so seeded Gaussian activations of the pages' shapes stand in for them):

* Q, K, V and dO are drawn i.i.d. N(0, 1) in fp32 with ``numpy.random.default_rng(seed)``,
  in the order Q, K, V, dO, each of shape [B, H, N, D].
* For bf16 workloads the fp32 draws are rounded to bf16 with round-to-nearest-even; the
  oracle consumes the exact bf16 values widened to fp64.
* seed = config * 10**6 + base_id * 10**5 + window * 10**3 + layer.
* Per-layer alphas of the learned-dilation workload are drawn
  ``default_rng(seed).uniform(lo, hi, n_layers)`` and rounded to fp32.

Two structured input sets serve as probes (values exact in bf16):

* ``staircase_inputs``: Q, K ~ N(0, 1); V ~ N(0, 1) except column 0, which holds
  (j mod 64) / 8 at position j; dO = the unit vector of column 0 at every position. The
  per-query contributions to d(alpha) then share one sign instead of cancelling.
* ``position_code_v``: V[j] holds binary codes of the position j (its bits and the bits of
  two odd multiples of j, modulo 2^bits), and a constant 1.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "seed_for",
    "normal_inputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "uniform_alphas",
    "random_alpha_grid",
    "staircase_inputs",
    "position_code_v",
]


def seed_for(config: int, base_id: int = 0, window: int = 0, layer: int = 0) -> int:
    """Seed of one (workload, base, window, layer) input set."""
    return int(config) * 10**6 + int(base_id) * 10**5 + int(window) * 10**3 + int(layer)


def normal_inputs(seed: int, shape, with_dout: bool = False):
    """Draw Q, K, V (and dO) ~ N(0, 1) as fp32 arrays of ``shape`` from one generator."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if not with_dout:
        return q, k, v
    do = rng.standard_normal(shape, dtype=np.float32)
    return q, k, v, do


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns.

    NaN inputs map to a quiet NaN; the test inputs are finite draws.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to the fp32 values they denote (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniform_alphas(seed: int, n: int, lo: float, hi: float) -> np.ndarray:
    """n per-layer alphas ~ U[lo, hi) rounded to fp32 (learned-dilation workload)."""
    return np.random.default_rng(seed).uniform(lo, hi, n).astype(np.float32)


def random_alpha_grid(seed: int, n: int, lo: float = 0.5, hi: float = 1.5) -> np.ndarray:
    """n random fp32 alphas in [lo, hi) for table sweeps."""
    return np.random.default_rng(seed).uniform(lo, hi, n).astype(np.float32)


def staircase_inputs(seed: int, shape):
    """Q, K, V, dO as fp32 arrays of ``shape`` [.., N, D]: Q, K and V drawn N(0, 1) from one
    generator (in that order); V[..., j, 0] = (j mod 64) / 8; dO = 1 in column 0, else 0."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    N = shape[-2]
    v[..., :, 0] = (np.arange(N) % 64).astype(np.float32) / 8.0
    do = np.zeros(shape, dtype=np.float32)
    do[..., :, 0] = 1.0
    return q, k, v, do


# odd multipliers of the position codes (any odd number permutes the residues mod 2^bits)
CODE_MULT = (1, 40503, 51749)


def position_code_v(N: int, D: int = 64, bits: int = 17) -> np.ndarray:
    """[N, D] fp32 (0/1 values): column c * bits + b (c < 3, b < bits) holds bit b of
    (j * CODE_MULT[c]) mod 2^bits for position j; the last column is 1; other columns 0."""
    if 3 * bits + 1 > D:
        raise ValueError("D too small for the codes")
    j = np.arange(N, dtype=np.int64)
    v = np.zeros((N, D), dtype=np.float32)
    for c, m in enumerate(CODE_MULT):
        code = (j * m) & ((1 << bits) - 1)
        for b in range(bits):
            v[:, c * bits + b] = (code >> b) & 1
    v[:, D - 1] = 1.0
    return v
