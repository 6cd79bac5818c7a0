"""Pins of the oracle's hand-derived backward (CPU only): torch fp64 autograd through the
independent dense formulations, and central finite differences of the oracle's own forward
(d alpha included)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from dense_reference import dense_augmented, dense_int_forward
from fibonacci_offset_dilated_amd.workloads import FIB_BASE

SMALL_FIB = FIB_BASE[:10]


def _inputs(seed, B, H, N, D=64):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, D)) for _ in range(4)]


@pytest.mark.parametrize("alpha", [np.float32(1.0), np.float32(0.7), np.float32(1.5)])
@pytest.mark.parametrize("W", [1, 6])
def test_int_backward_vs_autograd(alpha, W):
    q, k, v, do = _inputs(int(alpha * 10) + W, 1, 2, 70)
    dq, dk, dv, da = O.backward(q, k, v, do, W, alpha, SMALL_FIB, 10000.0, O.INT)
    qt, kt, vt = (torch.tensor(t, requires_grad=True) for t in (q, k, v))
    o, _ = dense_int_forward(qt, kt, vt, W, alpha, SMALL_FIB)
    (o * torch.as_tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=0, atol=1e-11)
    assert da == 0.0


@pytest.mark.parametrize("alpha", [np.float32(0.973), np.float32(1.0417), np.float32(1.5)])
@pytest.mark.parametrize("W", [4, 12])
def test_interp_backward_vs_autograd(alpha, W):
    q, k, v, do = _inputs(int(alpha * 1000) + W, 1, 2, 70)
    dq, dk, dv, da = O.backward(q, k, v, do, W, alpha, SMALL_FIB, 10000.0, O.INTERP)
    qt, kt, vt = (torch.tensor(t, requires_grad=True) for t in (q, k, v))
    at = torch.tensor(float(alpha), dtype=torch.float64, requires_grad=True)
    o, _ = dense_augmented(qt, kt, vt, W, at, SMALL_FIB)
    (o * torch.as_tensor(do)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(da, at.grad.item(), rtol=1e-10, atol=1e-10)
    *_, da2, sc = O.backward(q, k, v, do, W, alpha, SMALL_FIB, 10000.0, O.INTERP, return_scale=True)
    assert da2 == da and sc.sum_abs >= abs(da) and sc.sum_abs > 0
    # sqrt(sum t_i^2) <= sum |t_i| <= sqrt(n) sqrt(sum t_i^2); |t_i| <= a_i <= b_i
    assert sc.rss_query <= sc.sum_abs * (1 + 1e-12) and sc.sum_abs <= math.sqrt(2 * 70) * sc.rss_query * (1 + 1e-12)
    assert sc.rss_query <= sc.rss_entry * (1 + 1e-12) <= sc.rss_wide * (1 + 1e-12)


def _loss(q, k, v, do, W, alpha, mode):
    o, _ = O.forward(q, k, v, W, alpha, SMALL_FIB, 10000.0, mode)
    return float((o * do).sum())


@pytest.mark.parametrize("mode", [O.INT, O.INTERP])
def test_finite_differences_qkv(mode):
    q, k, v, do = _inputs(31 + mode, 1, 1, 60)
    alpha = np.float32(1.0417)
    W = 6
    dq, dk, dv, _ = O.backward(q, k, v, do, W, alpha, SMALL_FIB, 10000.0, mode)
    rng = np.random.default_rng(7)
    h = 1e-6
    for grad, idx in ((dq, 0), (dk, 1), (dv, 2)):
        u = rng.standard_normal(q.shape)
        args = [q, k, v]
        plus = [a.copy() for a in args]
        minus = [a.copy() for a in args]
        plus[idx] += h * u
        minus[idx] -= h * u
        fd = (_loss(*plus, do, W, alpha, mode) - _loss(*minus, do, W, alpha, mode)) / (2 * h)
        assert abs(fd - float((grad * u).sum())) < 1e-6 * max(1.0, abs(fd))


def test_finite_difference_alpha():
    # alpha chosen so that no alpha*f is within h*f of an integer, of W or of a query index
    q, k, v, do = _inputs(77, 1, 2, 120)
    W = 6
    for alpha in (np.float32(0.9731), np.float32(1.0417), np.float32(1.2389)):
        _, _, _, da = O.backward(q, k, v, do, W, alpha, SMALL_FIB, 10000.0, O.INTERP)
        a = float(alpha)
        h = 1e-7
        # forward at alpha +- h with the same integer parts: evaluate through the dense formulation
        # (the oracle takes fp32 alpha, too coarse for a finite difference of step 1e-7)
        def L(x):
            at = torch.tensor(x, dtype=torch.float64)
            o, _ = dense_augmented(q, k, v, W, at, SMALL_FIB)
            return float((o.numpy() * do).sum())
        # the dense formulation fixes c from alpha, so both sides share the table of alpha
        fd = (L(a + h) - L(a - h)) / (2 * h)
        assert abs(fd - da) < 1e-5 * max(1.0, abs(fd)), (alpha, fd, da)


def test_dalpha_bound_discriminates():
    """The dalpha bound of the GPU tests (gpu_util.dalpha_bound), computed from the oracle
    alone, is a small fraction of |dalpha| on the learned-dilation workload (B8 H8 N1024 bf16
    inputs, W 12; layers 0 and 7 are the two with the most cancellation among the 15 layers
    whose dalpha stands out of its rounding noise) and on the staircase probe, whose
    per-query contributions share one sign."""
    from gpu_util import dalpha_bound
    from fibonacci_offset_dilated_amd.synthetic import (bf16_bits_to_f32, f32_to_bf16_bits, normal_inputs, seed_for,
                                                        staircase_inputs, uniform_alphas)
    from fibonacci_offset_dilated_amd.workloads import BF16, BY_CONFIG, FIB_BASE, UNIFORM_ALPHA_RANGE, UNIFORM_ALPHA_SEED

    def exact_bf16(arrs):
        return [bf16_bits_to_f32(f32_to_bf16_bits(a)).astype(np.float64) for a in arrs]

    w = BY_CONFIG[3]
    al = uniform_alphas(UNIFORM_ALPHA_SEED, 16, *UNIFORM_ALPHA_RANGE)
    for layer in (0, 7):
        h = exact_bf16(normal_inputs(seed_for(3, 0, 12, layer), (w.B, w.H, w.N, w.D), with_dout=True))
        _, _, _, da, sc = O.backward(*h, 12, al[layer], FIB_BASE, 10000.0, O.INTERP, workers=8, return_scale=True)
        assert dalpha_bound(sc, BF16) < 0.05 * abs(da), (layer, dalpha_bound(sc, BF16) / abs(da))
    h = exact_bf16(staircase_inputs(77, (2, 4, 2048, 64)))
    _, _, _, da, sc = O.backward(*h, 12, np.float32(1.0417), FIB_BASE, 10000.0, O.INTERP, workers=8,
                                 return_scale=True)
    assert dalpha_bound(sc, BF16) < 0.01 * abs(da)
