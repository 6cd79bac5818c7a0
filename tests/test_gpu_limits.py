"""GPU parity at the size limits the index arithmetic has to survive, via the C ABI:
a 2^21-row head (16x the long-context length; row offsets beyond 2^31 bytes per tensor),
32768 heads of 32 rows (many workgroups, short sequences), and a 256-layer stack. Sampled
against the CPU oracle with the same bounds as the other parity tests.
"""
import numpy as np
import pytest
import torch

import fibonacci_offset_dilated_amd as F
import oracle as O
from fibonacci_offset_dilated_amd.workloads import BF16, F32, FIB_BASE, INT, INTERP
from gpu_util import TOL, grad_excess, host, inputs, maxabs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def huge_inputs():
    say("inputs B1 H1 N2097152 bf16 (+dO)")
    return inputs(31337, (1, 1, 1 << 21, 64), BF16, with_dout=True)


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_two_million_rows(huge_inputs, mode):
    N = 1 << 21
    a = np.float32(1.5)
    (q, q64), (k, k64), (v, v64), (do, d64) = huge_inputs
    say(f"N={N} mode={mode}: forward")
    o, lse = F.fwd(q, k, v, 12, a, FIB_BASE, 10000.0, mode)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5 + mode)
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(1470, 1500), rng.integers(0, N, 400),
                                     np.arange((1 << 20) - 20, (1 << 20) + 20), np.arange(N - 40, N)]))
    ro, rl = O.forward_rows(q64[0, 0], k64[0, 0], v64[0, 0], rows, 12, a, FIB_BASE, 10000.0, mode)
    eo, el = maxabs(host(o[0, 0])[rows], ro), maxabs(host(lse[0, 0])[rows], rl)
    say(f"  forward: max err O {eo:.3e} LSE {el:.3e}")
    assert eo <= TOL[BF16] and el <= TOL[BF16]
    say("  backward")
    dq, dk, dv, _ = F.bwd(q, k, v, o, lse, do, 12, a, FIB_BASE, 10000.0, mode)
    torch.cuda.synchronize()
    reach = 1481 + 12 + 2
    eg = 0.0
    for j0 in (0, (1 << 20) - 150, N - 300):
        j1 = min(N, j0 + 300)
        r = np.arange(j0, min(N, j1 + reach))
        rq, rk, rv, _ = O.backward(q64, k64, v64, d64, 12, a, FIB_BASE, 10000.0, mode, rows=r)
        eg = max(eg, grad_excess(host(dq[0, 0, j0:j1]), rq[0, 0, j0:j1], BF16),
                 grad_excess(host(dk[0, 0, j0:j1]), rk[0, 0, j0:j1], BF16),
                 grad_excess(host(dv[0, 0, j0:j1]), rv[0, 0, j0:j1], BF16))
    say(f"  backward: grad excess {eg:.3e}")
    assert eg <= TOL[BF16]


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
def test_many_heads(dtype):
    B, H, N = 64, 512, 32
    a = np.float32(0.75)
    say(f"B{B} H{H} N{N} dtype {dtype}")
    (q, q64), (k, k64), (v, v64), (do, d64) = inputs(4242 + dtype, (B, H, N, 64), dtype, with_dout=True)
    o, lse = F.fwd(q, k, v, 12, a, FIB_BASE, 10000.0, INTERP)
    dq, dk, dv, da = F.bwd(q, k, v, o, lse, do, 12, a, FIB_BASE, 10000.0, INTERP)
    torch.cuda.synchronize()
    picks = [(0, 0), (B - 1, H - 1), (17, 300), (40, 5), (63, 0), (0, 511)]
    sel = lambda x, b, h: x[b:b + 1, h:h + 1]  # noqa: E731
    eo = eg = 0.0
    for b, h in picks:
        ro, rl = O.forward(sel(q64, b, h), sel(k64, b, h), sel(v64, b, h), 12, a, FIB_BASE, 10000.0, INTERP)
        eo = max(eo, maxabs(host(o[b, h]), ro[0, 0]), maxabs(host(lse[b, h]), rl[0, 0]))
        rq, rk, rv, _ = O.backward(sel(q64, b, h), sel(k64, b, h), sel(v64, b, h), sel(d64, b, h), 12, a, FIB_BASE,
                                   10000.0, INTERP)
        eg = max(eg, grad_excess(host(dq[b, h]), rq[0, 0], dtype), grad_excess(host(dk[b, h]), rk[0, 0], dtype),
                 grad_excess(host(dv[b, h]), rv[0, 0], dtype))
    say(f"  max err O/LSE {eo:.3e}; grad excess {eg:.3e}")
    assert eo <= TOL[dtype] and eg <= TOL[dtype]


def test_256_layer_stack():
    L, B, H, N = 256, 1, 2, 200
    al = np.random.default_rng(9).uniform(0.5, 1.5, L).astype(np.float32)
    say(f"L{L} B{B} H{H} N{N}")
    (q, _), (k, _), (v, _) = inputs(777, (L * B, H, N, 64), BF16)
    q, k, v = (t.view(L, B, H, N, 64) for t in (q, k, v))
    o, lse = F.fwd_layers(q, k, v, 12, al, FIB_BASE, 10000.0, INTERP)
    od, _ = F.decode_layers(q[:, :, :, -1].contiguous(), k, v, 12, al, FIB_BASE, 10000.0, INTERP)
    torch.cuda.synchronize()
    e = 0.0
    for l in (0, 1, 127, 200, 255):
        os_, ls_ = F.fwd(q[l], k[l], v[l], 12, al[l], FIB_BASE, 10000.0, INTERP)
        ds_, _ = F.decode(q[l, :, :, -1].contiguous(), k[l], v[l], 12, al[l], FIB_BASE, 10000.0, INTERP)
        torch.cuda.synchronize()
        e = max(e, maxabs(host(o[l]), host(os_)), maxabs(host(lse[l]), host(ls_)))
        assert torch.equal(od[l], ds_)
    say(f"  stack vs single-layer calls {e:.3e}")
    assert e <= TOL[BF16]
