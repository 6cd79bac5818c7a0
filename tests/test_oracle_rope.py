"""Pins of the oracle's RoPE (CPU only): closed forms, complex-multiplication formulation,
norm preservation and the relative-position identity."""
import math

import numpy as np
import torch

import oracle as O
from dense_reference import rope_complex


def test_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((1, 64))
    assert np.array_equal(O.rope(x, 10000.0), x)


def test_closed_form_unit_vectors():
    # D = 4, theta = 10000: omega = (1, 10000^(-1/2) = 0.01). At position p the pair (0, 2)
    # rotates by p rad and the pair (1, 3) by 0.01 p rad.
    x = np.zeros((3, 4))
    x[:, 0] = 1.0
    x[:, 3] = 1.0
    y = O.rope(x, 10000.0)
    for p in range(3):
        np.testing.assert_allclose(y[p], [math.cos(p), -math.sin(0.01 * p), math.sin(p), math.cos(0.01 * p)],
                                   rtol=0, atol=1e-15)


def test_matches_complex_multiplication():
    x = np.random.default_rng(1).standard_normal((2, 700, 64))
    a = O.rope(x, 10000.0)
    b = rope_complex(torch.as_tensor(x), 10000.0).numpy()
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_norm_and_inverse():
    x = np.random.default_rng(2).standard_normal((131, 64))
    y = O.rope(x, 500.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(O.rope_inverse(y, 500.0), x, rtol=0, atol=1e-13)


def test_relative_identity():
    rng = np.random.default_rng(3)
    q = rng.standard_normal(64)
    k = rng.standard_normal(64)
    N = 2000
    Q = np.tile(q, (N, 1))
    K = np.tile(k, (N, 1))
    Qr = O.rope(Q, 10000.0)
    Kr = O.rope(K, 10000.0)
    for i, j in ((5, 3), (1999, 1000), (987, 0), (40, 40)):
        lhs = Qr[i] @ Kr[j]
        rhs = O.rope(np.tile(q, (i - j + 1, 1)), 10000.0)[i - j] @ k
        assert abs(lhs - rhs) < 1e-10
