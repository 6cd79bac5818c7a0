"""Pins of the oracle's hand-derived backward (CPU only): torch fp64 autograd through the
independent dense formulations, and central finite differences of the oracle's own forward
(d alpha included)."""
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
    *_, da2, dabs = O.backward(q, k, v, do, W, alpha, SMALL_FIB, 10000.0, O.INTERP, return_abs=True)
    assert da2 == da and dabs >= abs(da) and dabs > 0


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
