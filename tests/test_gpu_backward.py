"""GPU parity of the backward pass (dQ, dK, dV, dalpha) against the CPU oracle, via the C ABI.

Bounds: |error| on dQ, dK, dV within 1e-4 (fp32) / 2e-2 (bf16) plus one ulp of the input
dtype at the reference value (see gpu_util.grad_excess); |error| on dalpha within the bound
derived from the rounding of its per-query parts (gpu_util.dalpha_bound), and, where the
per-query contributions do not cancel, within 2e-2 of |dalpha|. The GPU uses its own bf16 O
(for Delta) and fp32 LSE from the forward, as a training step would; the oracle computes exact
gradients.
"""
import os

import numpy as np
import pytest
import torch

import fibonacci_offset_dilated_amd as F
import oracle as O
from fibonacci_offset_dilated_amd.synthetic import seed_for, uniform_alphas
from fibonacci_offset_dilated_amd.workloads import (BF16, BY_CONFIG, F32, FIB_BASE, INT, INTERP, POW2_BASE,
                                                    UNIFORM_ALPHA_RANGE, UNIFORM_ALPHA_SEED)
from gpu_util import TOL, dalpha_check, grad_excess, host, inputs, maxabs, say

pytestmark = pytest.mark.gpu
WORKERS = min(16, len(os.sched_getaffinity(0)))


def gpu_grads(qkvd, W, alpha, base, mode):
    (q, _), (k, _), (v, _), (do, _) = qkvd
    o, lse = F.fwd(q, k, v, W, alpha, base, 10000.0, mode)
    dq, dk, dv, da = F.bwd(q, k, v, o, lse, do, W, alpha, base, 10000.0, mode)
    torch.cuda.synchronize()
    return dq, dk, dv, da


def check(qkvd, W, alpha, base, mode, dtype):
    (_, q64), (_, k64), (_, v64), (_, d64) = qkvd
    dq, dk, dv, da = gpu_grads(qkvd, W, alpha, base, mode)
    rq, rk, rv, ra, rsc = O.backward(q64, k64, v64, d64, W, alpha, base, 10000.0, mode, workers=WORKERS,
                                     return_scale=True)
    eq, ek, ev = grad_excess(host(dq), rq, dtype), grad_excess(host(dk), rk, dtype), grad_excess(host(dv), rv, dtype)
    got_a = float(da.item())
    say(f"  dQ {eq:.2e} dK {ek:.2e} dV {ev:.2e}")
    assert max(eq, ek, ev) <= TOL[dtype], (eq, ek, ev)
    if mode == INT:
        assert got_a == 0.0
    else:
        dalpha_check(got_a, ra, rsc, dtype)
    return got_a, ra


@pytest.mark.parametrize("layer", range(16))
def test_learned_dilation_layers_backward(layer):
    w = BY_CONFIG[3]
    a = uniform_alphas(UNIFORM_ALPHA_SEED, 16, *UNIFORM_ALPHA_RANGE)[layer]
    say(f"learned dilation bwd B8H8N1024 bf16 W=12 layer={layer} alpha={a}")
    qkvd = inputs(seed_for(3, 0, 12, layer), (w.B, w.H, w.N, w.D), BF16, with_dout=True)
    check(qkvd, 12, a, FIB_BASE, INTERP, BF16)


EDGE = [
    (1, 1, 1, 1, 1.0, FIB_BASE),
    (1, 2, 2, 12, 1.0, FIB_BASE),
    (2, 1, 65, 6, 0.7, FIB_BASE),
    (1, 2, 200, 16, 1.3, FIB_BASE),
    (1, 1, 300, 17, 1.07, FIB_BASE),
    (1, 1, 257, 40, 0.93, POW2_BASE),
    (1, 2, 130, 130, 1.0, FIB_BASE),
    (1, 1, 100, 12, 40.0, FIB_BASE),
    (1, 1, 1100, 12, 1.5, FIB_BASE),
]


@pytest.mark.parametrize("dtype", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("case", EDGE, ids=[f"B{c[0]}H{c[1]}N{c[2]}W{c[3]}a{c[4]}" for c in EDGE])
def test_backward_edge_shapes(case, mode, dtype):
    B, H, N, W, alpha, base = case
    say("bwd edge", case, mode, dtype)
    qkvd = inputs(2000 + N + W, (B, H, N, 64), dtype, with_dout=True)
    check(qkvd, W, np.float32(alpha), base, mode, dtype)


# cases aimed at the LDS-ring query-side kernel (bf16, W <= 16): segment edges, ring reach,
# far entries, partial steps, 4-wave instances
RING_BWD = [
    # (B, H, N, W, alpha, base)
    (1, 1, 10000, 12, 1.5, FIB_BASE),          # many segments, far entries 566/915/1480
    (1, 3, 5000, 16, 1.0, (1, 2, 512, 513, 700)),  # distances 512 (ring) and 513, 700 (global)
    (2, 1, 4100, 1, 1.5, POW2_BASE),           # W = 1, far rows up to 3072
    (1, 2, 70, 6, 0.5, FIB_BASE),              # one partial step
    (3, 5, 1500, 10, 1.3, FIB_BASE),
    (1, 1, 2000, 12, 1.0001, (1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 511, 512, 610)),
    (1, 2, 3001, 7, 1.37, FIB_BASE),           # interpolation weights of every size, ragged end
    (2, 2, 700, 12, 1.45, FIB_BASE),           # one far entry (c = 547) read by few queries
]


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("case", RING_BWD,
                         ids=[f"B{c[0]}H{c[1]}N{c[2]}W{c[3]}a{c[4]}n{len(c[5])}" for c in RING_BWD])
def test_backward_ring_cases(case, mode):
    B, H, N, W, alpha, base = case
    say("bwd ring", case, mode)
    qkvd = inputs(5000 + N + W, (B, H, N, 64), BF16, with_dout=True)
    check(qkvd, W, np.float32(alpha), base, mode, BF16)


@pytest.fixture(scope="module")
def long_inputs():
    w = BY_CONFIG[5]
    say("long context inputs B1H32N131072 bf16 (+dO)")
    return inputs(seed_for(5, 0, 12, 15), (w.B, w.H, w.N, w.D), BF16, with_dout=True)


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_long_context_backward_sampled(long_inputs, mode):
    """dQ on sampled query rows; dK/dV on key ranges, from the oracle restricted to the queries
    that read those keys; dalpha over the whole call."""
    w = BY_CONFIG[5]
    a = F.schedule_alpha(F.SCHED_LINEAR, 15, 16)
    say(f"long context bwd N=131072 H=32 alpha={a} mode={mode}")
    dq, dk, dv, da = gpu_grads(long_inputs, 12, a, FIB_BASE, mode)
    (_, q64), (_, k64), (_, v64), (_, d64) = long_inputs
    reach = 1481 + 12 + 2
    # heads 0 and 21: the start, the middle and the end; every other head: one key range
    ranges = [(h, j0) for h in (0, 21) for j0 in (0, 60000, w.N - 300)]
    ranges += [(h, (h * 4099) % (w.N - 300)) for h in range(w.H) if h not in (0, 21)]
    for h, j0 in ranges:
        j1 = min(w.N, j0 + 300)
        rows = np.arange(j0, min(w.N, j1 + reach))
        rq, rk, rv, _ = O.backward(q64[:, h:h + 1], k64[:, h:h + 1], v64[:, h:h + 1], d64[:, h:h + 1], 12, a,
                                   FIB_BASE, 10000.0, mode, rows=rows)
        eq = grad_excess(host(dq[0, h, j0:j1]), rq[0, 0, j0:j1], BF16)
        ek = grad_excess(host(dk[0, h, j0:j1]), rk[0, 0, j0:j1], BF16)
        ev = grad_excess(host(dv[0, h, j0:j1]), rv[0, 0, j0:j1], BF16)
        say(f"  head {h} rows {j0}:{j1} dQ {eq:.2e} dK {ek:.2e} dV {ev:.2e}")
        assert max(eq, ek, ev) <= TOL[BF16]
    if mode == INT:
        assert float(da.item()) == 0.0
    else:
        # dalpha over 4 of the heads at full length: the same kernels on a 4-head call
        hs = [0, 9, 18, 27]
        sub = [t[:, hs].contiguous() for t, _ in long_inputs]
        o4, l4 = F.fwd(sub[0], sub[1], sub[2], 12, a, FIB_BASE, 10000.0, mode)
        _, _, _, da4 = F.bwd(sub[0], sub[1], sub[2], o4, l4, sub[3], 12, a, FIB_BASE, 10000.0, mode)
        _, _, _, ra, rsc = O.backward(q64[:, hs], k64[:, hs], v64[:, hs], d64[:, hs], 12, a, FIB_BASE, 10000.0,
                                      mode, workers=WORKERS, return_scale=True)
        dalpha_check(float(da4.item()), ra, rsc, BF16, label="dalpha(4 heads)")
        # the sum does not cancel here: also within 2e-2 of |dalpha|
        assert abs(float(da4.item()) - ra) <= 2e-2 * abs(ra)


# Long segments (at least 8 steps) with the entries just past the ring reach (384, 640], at
# the edges of that range, after none or 15 covered entries: the integer query side's dQ on
# the first three steps of several segments (where the far rows precede the segment), random
# rows and the end, against the oracle.
FAR_EDGE_BWD = [
    # (B, H, N, W, alpha, base)
    (1, 16, 40000, 12, 1.5, FIB_BASE),           # far entries 566, 915 and 1480
    (1, 8, 70000, 16, 1.0, (1, 2, 640, 1024)),
    (1, 8, 70000, 16, 1.0, (1, 2, 385, 641)),
    (1, 8, 60000, 12, 1.0, tuple(range(20, 380, 25)) + (600, 900)),  # 15 covered
    (1, 8, 60000, 12, 1.0, (1, 2, 500)),
]


@pytest.mark.parametrize("case", FAR_EDGE_BWD, ids=[f"B{c[0]}H{c[1]}N{c[2]}W{c[3]}a{c[4]}n{len(c[5])}" for c in FAR_EDGE_BWD])
def test_far_entries_long_segments_backward(case):
    from test_gpu_forward import ring_segment_len

    B, H, N, W, alpha, base = case
    alpha = np.float32(alpha)
    seg = ring_segment_len(B * H, N)
    assert seg >= 8 * 128
    say("far entries, long segments, backward", case, "segment rows", seg)
    qkvd = inputs(6000 + N + W, (B, H, N, 64), BF16, with_dout=True)
    dq, _, _, da = gpu_grads(qkvd, W, alpha, base, INT)
    n_seg = -(-N // seg)
    firsts = [seg * k for k in sorted({0, 1, 2, n_seg // 2, n_seg - 1})]
    rng = np.random.default_rng(N + W + 1)
    rows = np.unique(np.concatenate([np.arange(s, min(s + 3 * 128 + 8, N)) for s in firsts]
                                    + [rng.integers(0, N, 100), np.arange(N - 24, N)]))
    (_, q64), (_, k64), (_, v64), (_, d64) = qkvd
    eq = 0.0
    for b, h in [(0, 0), (B - 1, H - 1)]:
        rq, _, _, _ = O.backward(q64[b:b + 1, h:h + 1], k64[b:b + 1, h:h + 1], v64[b:b + 1, h:h + 1],
                                 d64[b:b + 1, h:h + 1], W, alpha, base, 10000.0, INT, rows=rows)
        eq = max(eq, grad_excess(host(dq[b, h])[rows], rq[0, 0][rows], BF16))
    say(f"  dQ {eq:.2e} over {len(rows)} rows")
    assert eq <= TOL[BF16]
    assert float(da.item()) == 0.0


def _sixteen_heads(N, seed):
    """16-head inputs whose heads 0 and 15 hold seeded N(0, 1) draws and the rest zeros (their
    gradients and d(alpha) parts are 0), with the fp64 copies of the two live heads."""
    live = inputs(seed, (1, 2, N, 64), BF16, with_dout=True)
    out = []
    for t, t64 in live:
        z = torch.zeros((1, 16, N, 64), dtype=t.dtype, device=t.device)
        z[:, 0], z[:, 15] = t[:, 0], t[:, 1]
        out.append((z, t64))
    return out


def test_interp_backward_far_rows_rotated():
    """Interpolated backward where the query side reads its far K rows as rotated rows that it
    wrote itself (16 heads of 65536 rows: segments of 2048 rows, far distances 549 and 889 at
    alpha 0.9, so each workgroup first rotates the rows before its segment): every row of the
    two live heads against the oracle, and dalpha."""
    N, a = 65536, np.float32(0.9)
    say(f"bwd rotated far rows B1H16N{N} alpha={a}")
    qkvd = _sixteen_heads(N, 7700)
    dq, dk, dv, da = gpu_grads(qkvd, 12, a, FIB_BASE, INTERP)
    (_, q64), (_, k64), (_, v64), (_, d64) = qkvd
    rq, rk, rv, ra, rsc = O.backward(q64, k64, v64, d64, 12, a, FIB_BASE, 10000.0, INTERP, workers=WORKERS,
                                     return_scale=True)
    for h, hr in ((0, 0), (15, 1)):
        eq = grad_excess(host(dq[0, h]), rq[0, hr], BF16)
        ek = grad_excess(host(dk[0, h]), rk[0, hr], BF16)
        ev = grad_excess(host(dv[0, h]), rv[0, hr], BF16)
        say(f"  head {h} dQ {eq:.2e} dK {ek:.2e} dV {ev:.2e}")
        assert max(eq, ek, ev) <= TOL[BF16]
    for h in range(1, 15):
        assert not dq[0, h].any() and not dk[0, h].any() and not dv[0, h].any()
    dalpha_check(float(da.item()), ra, rsc, BF16)


def test_interp_backward_far_rows_rotated_device_alpha():
    """The same path with alpha in device memory (16 heads of 131072 rows, alpha 0.9 in the
    declared range [0.85, 0.95]): gradients and dalpha against the host-alpha call, whose
    kernels read the same table."""
    N, a = 131072, np.float32(0.9)
    say(f"bwd rotated far rows, device alpha, B1H16N{N}")
    qkvd = _sixteen_heads(N, 7800)
    (q, _), (k, _), (v, _), (do, _) = qkvd
    o, lse = F.fwd(q, k, v, 12, a, FIB_BASE, 10000.0, INTERP)
    ref = F.bwd(q, k, v, o, lse, do, 12, a, FIB_BASE, 10000.0, INTERP)
    ad = torch.tensor([float(a)], dtype=torch.float32, device="cuda")
    got = F.bwd_dev(q, k, v, o, lse, do, 12, ad, (0.85, 0.95), FIB_BASE, 10000.0, INTERP)
    torch.cuda.synchronize()
    for name, x, y in zip(("dQ", "dK", "dV"), ref[:3], got[:3]):
        e = maxabs(host(x), host(y))
        say(f"  {name} device vs host alpha {e:.2e}")
        assert e <= TOL[BF16], name
    ea = abs(float(got[3].item()) - float(ref[3].item()))
    say(f"  dalpha device {float(got[3].item()):.7g} host {float(ref[3].item()):.7g}")
    assert ea <= 1e-3 * abs(float(ref[3].item()))


def test_backward_deterministic():
    say("bwd determinism")
    qkvd = inputs(9, (1, 4, 2500, 64), BF16, with_dout=True)
    r1 = gpu_grads(qkvd, 12, np.float32(1.21), FIB_BASE, INTERP)
    r2 = gpu_grads(qkvd, 12, np.float32(1.21), FIB_BASE, INTERP)
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_dalpha_output_is_overwritten(mode):
    """dalpha is written, not accumulated: a buffer holding NaN before the call gets 0
    (integer offsets) or the same bits as a call into a fresh buffer (interpolated), for one
    layer and for a stack of layers, on the ring kernels (bf16, W 12, two far entries)."""
    B, H, N, W, alpha = 2, 2, 1500, 12, np.float32(1.04)
    say("dalpha overwrite", (B, H, N, W), "mode", mode)
    (q, _), (k, _), (v, _), (do, _) = inputs(9911, (B, H, N, 64), BF16, with_dout=True)
    o, lse = F.fwd(q, k, v, W, alpha, FIB_BASE, 10000.0, mode)
    _, _, _, fresh = F.bwd(q, k, v, o, lse, do, W, alpha, FIB_BASE, 10000.0, mode)
    stale = torch.full((1,), float("nan"), dtype=torch.float32, device=q.device)
    F.bwd(q, k, v, o, lse, do, W, alpha, FIB_BASE, 10000.0, mode, dalpha=stale)
    torch.cuda.synchronize()
    got, ref = host(stale)[0], host(fresh)[0]
    if mode == INT:
        assert got == 0.0 and ref == 0.0
    else:
        assert np.isfinite(got) and got == ref
    L = 3
    al = np.array([1.04, 0.97, 1.02], dtype=np.float32)
    qs, ks, vs, ds = (t.unsqueeze(0).expand(L, -1, -1, -1, -1).contiguous() for t in (q, k, v, do))
    os_, ls = F.fwd_layers(qs, ks, vs, W, al, FIB_BASE, 10000.0, mode)
    stale_l = torch.full((L,), float("nan"), dtype=torch.float32, device=q.device)
    F.bwd_layers(qs, ks, vs, os_, ls, ds, W, al, FIB_BASE, 10000.0, mode, dalpha=stale_l)
    single = []
    for l in range(L):
        o1, l1 = F.fwd(q, k, v, W, al[l], FIB_BASE, 10000.0, mode)
        single.append(F.bwd(q, k, v, o1, l1, do, W, al[l], FIB_BASE, 10000.0, mode)[3])
    torch.cuda.synchronize()
    got_l = host(stale_l)
    if mode == INT:
        assert np.all(got_l == 0.0)
    else:
        ref_l = np.array([host(s)[0] for s in single])
        assert np.all(np.isfinite(got_l))
        # the stack may split a layer's table differently from the single call (fp32 order)
        assert np.allclose(got_l, ref_l, rtol=1e-2, atol=1e-2 * np.abs(ref_l).max()), (got_l, ref_l)


STAIR = [(2, 4, 2048, 1.0417), (1, 2, 3000, 1.37), (1, 1, 20000, 1.5)]


@pytest.mark.parametrize("case", STAIR, ids=[f"B{c[0]}H{c[1]}N{c[2]}a{c[3]}" for c in STAIR])
def test_dalpha_without_cancellation(case):
    """Staircase probe (synthetic.staircase_inputs): the per-query contributions to dalpha
    share one sign, so the bound is far below |dalpha|; dalpha must also be within 2e-2 of
    |dalpha| (bf16, W 12, interpolated offsets, ring kernels)."""
    from fibonacci_offset_dilated_amd.synthetic import staircase_inputs
    from gpu_util import to_device
    B, H, N, a = case
    say("dalpha staircase", case)
    qkvd = [to_device(x, BF16) for x in staircase_inputs(77, (B, H, N, 64))]
    got, ref = check(qkvd, 12, np.float32(a), FIB_BASE, INTERP, BF16)
    assert abs(got - ref) <= 2e-2 * abs(ref)
