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
from gpu_util import TOL, dalpha_check, grad_excess, host, inputs, maxabs, say

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
    rq, rk, rv, ra, rsc = O.backward(q64, k64, v64, d64, 12, np.float32(1.21), FIB_BASE, 10000.0, mode,
                                     workers=8, return_scale=True)
    e = max(grad_excess(host(qq.grad), rq, dtype), grad_excess(host(kk.grad), rk, dtype),
            grad_excess(host(vv.grad), rv, dtype))
    say(f"autograd mode {mode} dtype {dtype}: grad excess {e:.2e}")
    assert e <= TOL[dtype]
    if mode == INT:
        assert float(alpha.grad.item()) == 0.0
    else:
        dalpha_check(float(alpha.grad.item()), ra, rsc, dtype)


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
    _, _, _, ra, rsc = O.backward(q64, k64, v64, d64, 12, a, FIB_BASE, 10000.0, INTERP, workers=8,
                                  return_scale=True)
    dmap = 0.5 * (1.0 - np.tanh(0.3) ** 2)
    # (the map itself is evaluated in fp32 by torch: its relative error adds 2^-20 of |dtheta|)
    dalpha_check(float(layer.theta.grad.item()), ra * dmap, rsc, F32, factor=dmap * (1 + 2.0 ** -20),
                 label="dtheta")


@pytest.mark.parametrize("learned", [False, True], ids=["static-int", "learned-interp"])
def test_attention_layer_module(learned):
    """FibSparseSelfAttention (fp32): output and gradients of x and of both projections against
    an fp64 composition of the projections with the oracle's forward and backward. Bound:
    the op's 1e-4 propagated through a projection row (|W| <= 1/sqrt(512), 512 terms: at most
    512 * 0.0442 * 1e-4 = 2.3e-3), so 2.5e-3 on outputs and gradients."""
    from fibonacci_offset_dilated_amd.autograd import FibSparseSelfAttention
    torch.manual_seed(11)
    B, N, C, H = 2, 300, 512, 8
    layer = FibSparseSelfAttention(C, H, 12, "learned" if learned else 1.21).cuda()
    if learned:
        with torch.no_grad():
            layer.dilation.theta.fill_(0.4)
    rng = np.random.default_rng(12)
    x64 = rng.standard_normal((B, N, C))
    dy64 = rng.standard_normal((B, N, C))
    x = torch.from_numpy(x64.astype(np.float32)).cuda().requires_grad_(True)
    y = layer(x)
    y.backward(torch.from_numpy(dy64.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    # fp64 reference
    x64 = x.detach().double().cpu().numpy()
    wqkv = layer.qkv.weight.detach().double().cpu().numpy()
    wo = layer.out.weight.detach().double().cpu().numpy()
    if learned:
        a = np.float32(layer.dilation.alpha().item())
        mode = INTERP
    else:
        a = np.float32(1.21)
        mode = INT
    qkv = (x64 @ wqkv.T).reshape(B, N, 3, H, 64).transpose(2, 0, 3, 1, 4)
    q, k, v = qkv[0], qkv[1], qkv[2]
    o, _ = O.forward(q, k, v, 12, a, FIB_BASE, 10000.0, mode, workers=8)
    o2 = o.transpose(0, 2, 1, 3).reshape(B, N, C)
    y_ref = o2 @ wo.T
    do2 = dy64 @ wo
    dwo = np.einsum("bni,bnj->ij", dy64, o2)
    do = do2.reshape(B, N, H, 64).transpose(0, 2, 1, 3)
    dq, dk, dv, da, dsc = O.backward(q, k, v, do, 12, a, FIB_BASE, 10000.0, mode, workers=8, return_scale=True)
    dqkv = np.stack([dq, dk, dv]).transpose(1, 3, 0, 2, 4).reshape(B, N, 3 * C)
    dx = dqkv @ wqkv
    dwqkv = np.einsum("bni,bnj->ij", dqkv, x64)
    e = {"y": maxabs(host(y), y_ref), "dx": maxabs(host(x.grad), dx),
         "dWqkv": maxabs(host(layer.qkv.weight.grad), dwqkv), "dWo": maxabs(host(layer.out.weight.grad), dwo)}
    say(f"attention layer (learned={learned}): {e}")
    assert max(e.values()) <= 2.5e-3
    if learned:
        th = float(layer.dilation.theta.item())
        dmap = 0.5 * (1.0 - np.tanh(th) ** 2)
        dalpha_check(float(layer.dilation.theta.grad.item()), da * dmap, dsc, F32, factor=dmap * (1 + 2.0 ** -20),
                     label="dtheta")
