"""GPU tests of the torch.autograd wrapper: gradients through the C ABI equal the backward
entry point's and the oracle's; the Learned-schedule parameter receives dalpha times the
derivative of its map."""
import numpy as np
import pytest
import torch

import fibonacci_offset_dilated_amd as F
import oracle as O
from fibonacci_offset_dilated_amd.autograd import LearnedDilation, fib_sparse_attention
from fibonacci_offset_dilated_amd.workloads import BF16, F32, FIB_BASE, INT, INTERP
from gpu_util import TOL, TOL_DALPHA, grad_excess, host, inputs, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("dtype", [F32, BF16], ids=["f32", "bf16"])
def test_autograd_matches_backward_entry_point_and_oracle(mode, dtype):
    (q, q64), (k, k64), (v, v64), (do, d64) = inputs(4242, (2, 3, 700, 64), dtype, with_dout=True)
    alpha = torch.tensor([1.21], dtype=torch.float32, device="cuda", requires_grad=True)
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = fib_sparse_attention(qq, kk, vv, alpha, 12, FIB_BASE, 10000.0, mode)
    (o.float() * do.float()).sum().backward()
    torch.cuda.synchronize()
    # the same kernels called directly
    of, lf = F.fwd(q, k, v, 12, np.float32(1.21), FIB_BASE, 10000.0, mode)
    dq, dk, dv, da = F.bwd(q, k, v, of, lf, do, 12, np.float32(1.21), FIB_BASE, 10000.0, mode)
    assert torch.equal(o.detach(), of)
    assert torch.equal(qq.grad, dq) and torch.equal(kk.grad, dk) and torch.equal(vv.grad, dv)
    assert alpha.grad is not None and float(alpha.grad.item()) == float(da.item())
    # and the oracle
    rq, rk, rv, ra, rabs = O.backward(q64, k64, v64, d64, 12, np.float32(1.21), FIB_BASE, 10000.0, mode,
                                      workers=8, return_abs=True)
    e = max(grad_excess(host(qq.grad), rq, dtype), grad_excess(host(kk.grad), rk, dtype),
            grad_excess(host(vv.grad), rv, dtype))
    ea = abs(float(alpha.grad.item()) - ra) / max(rabs, 1e-30)
    say(f"autograd mode {mode} dtype {dtype}: grad excess {e:.2e}, dalpha {float(alpha.grad.item()):.6g} "
        f"vs {ra:.6g} rel {ea:.2e}")
    assert e <= TOL[dtype]
    if mode == INT:
        assert float(alpha.grad.item()) == 0.0
    else:
        assert ea <= TOL_DALPHA[dtype]


def test_learned_dilation_theta_gradient():
    (q, q64), (k, k64), (v, v64), (do, d64) = inputs(777, (1, 2, 900, 64), F32, with_dout=True)
    layer = LearnedDilation().cuda()
    with torch.no_grad():
        layer.theta.fill_(0.3)
    o = layer(q, k, v, 12, FIB_BASE)
    (o * do).sum().backward()
    torch.cuda.synchronize()
    a = np.float32(1.0 + 0.5 * np.tanh(np.float32(0.3)))
    assert np.float32(layer.alpha().item()) == np.float32(1.0 + 0.5 * torch.tanh(torch.tensor(0.3)).item())
    _, _, _, ra, rabs = O.backward(q64, k64, v64, d64, 12, a, FIB_BASE, 10000.0, INTERP, workers=8,
                                   return_abs=True)
    want = ra * 0.5 * (1.0 - np.tanh(0.3) ** 2)
    got = float(layer.theta.grad.item())
    say(f"dtheta {got:.6g} vs {want:.6g}")
    assert abs(got - want) <= TOL_DALPHA[F32] * rabs * 0.5 + 1e-9
