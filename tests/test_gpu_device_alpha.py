"""GPU parity of the device-alpha entry points (alpha read from device memory, offset table
built on the GPU) against the CPU oracle and the host-alpha entry points, via the C ABI.

The device-alpha launch picks kernel instances for a whole alpha range and clamps alpha into
it, so the cases cover a tight range (lo = hi = alpha), the Learned schedule's [0.5, 1.5],
alpha outside the range (the result is the one at the clamped alpha), the LDS-ring kernels
(bf16, W <= 16) and the general kernels (fp32, wide windows). Bounds are the ones of the
forward, backward and decode tests: the two launches may split the table differently over
the kernel's covered and far slots, which changes only the order of fp32 sums.
"""
import os

import numpy as np
import pytest
import torch

import fibonacci_offset_dilated_amd as F
import oracle as O
from fibonacci_offset_dilated_amd.autograd import fib_sparse_attention
from fibonacci_offset_dilated_amd.synthetic import random_alpha_grid
from fibonacci_offset_dilated_amd.workloads import BF16, F32, FIB_BASE, INT, INTERP, POW2_BASE
from gpu_util import TOL, dalpha_check, grad_excess, host, inputs, maxabs, say

pytestmark = pytest.mark.gpu
WORKERS = min(16, len(os.sched_getaffinity(0)))
LEARNED = (0.5, 1.5)


def dev_alpha(a):
    return torch.tensor([float(a)], dtype=torch.float32, device="cuda")


def clamp(a, rng):
    return np.float32(min(max(np.float32(a), np.float32(rng[0])), np.float32(rng[1])))


FWD = [
    # (B, H, N, W, alpha, range, base, dtype)
    (2, 4, 3000, 12, 1.0, (1.0, 1.0), FIB_BASE, BF16),        # ring, tight range
    (2, 4, 3000, 12, 1.37, LEARNED, FIB_BASE, BF16),           # ring, Learned range
    (1, 2, 5000, 12, 0.5, LEARNED, FIB_BASE, BF16),            # alpha at the range's low end
    (1, 2, 5000, 12, 1.5, LEARNED, FIB_BASE, BF16),            # ... and high end
    (1, 3, 4100, 16, 1.0, (0.8, 1.2), (1, 2, 512, 513, 700), BF16),  # ring edge, far rows
    (2, 1, 4100, 1, 1.5, (1.0, 1.5), POW2_BASE, BF16),         # W = 1
    (1, 2, 70, 6, 0.77, LEARNED, FIB_BASE, BF16),              # one partial step
    (2, 3, 1000, 12, 1.21, LEARNED, FIB_BASE, F32),            # general kernel
    (1, 2, 1500, 40, 0.93, (0.5, 2.0), POW2_BASE, BF16),       # general kernel (wide window)
    (1, 1, 100, 12, 40.0, (1.0, 64.0), FIB_BASE, BF16),        # every offset beyond N
]


def fwd_ids(c):
    return f"B{c[0]}H{c[1]}N{c[2]}W{c[3]}a{c[4]}r{c[5][0]}-{c[5][1]}n{len(c[6])}-{'bf16' if c[7] else 'f32'}"


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("case", FWD, ids=[fwd_ids(c) for c in FWD])
def test_forward_device_alpha(case, mode):
    B, H, N, W, alpha, rng, base, dtype = case
    a = np.float32(alpha)
    say("fwd_dev", fwd_ids(case), "mode", mode)
    (q, q64), (k, k64), (v, v64) = inputs(8100 + N + W, (B, H, N, 64), dtype)
    o, lse = F.fwd_dev(q, k, v, W, dev_alpha(a), rng, base, 10000.0, mode)
    oh, lh = F.fwd(q, k, v, W, a, base, 10000.0, mode)
    torch.cuda.synchronize()
    ro, rl = O.forward(q64, k64, v64, W, a, base, 10000.0, mode, workers=WORKERS)
    eo, el = maxabs(host(o), ro), maxabs(host(lse), rl)
    ho, hl = maxabs(host(o), host(oh)), maxabs(host(lse), host(lh))
    say(f"  vs oracle O {eo:.3e} LSE {el:.3e}; vs host-alpha call O {ho:.3e} LSE {hl:.3e}")
    assert eo <= TOL[dtype] and el <= TOL[dtype]
    assert ho <= TOL[dtype] and hl <= TOL[dtype]


BWD = [
    (2, 3, 1024, 12, 1.21, LEARNED, FIB_BASE, BF16),
    (1, 1, 10000, 12, 1.5, LEARNED, FIB_BASE, BF16),           # far entries up to 1481
    (1, 2, 3001, 7, 1.37, (1.3, 1.4), FIB_BASE, BF16),
    (1, 3, 4100, 16, 1.0, (0.8, 1.2), (1, 2, 512, 513, 700), BF16),
    (2, 2, 700, 12, 0.61, LEARNED, FIB_BASE, F32),             # general kernel
    (1, 1, 257, 40, 0.93, (0.5, 2.0), POW2_BASE, BF16),        # general kernel (wide window)
]


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("case", BWD, ids=[fwd_ids(c) for c in BWD])
def test_backward_device_alpha(case, mode):
    B, H, N, W, alpha, rng, base, dtype = case
    a = np.float32(alpha)
    say("bwd_dev", fwd_ids(case), "mode", mode)
    (q, q64), (k, k64), (v, v64), (do, d64) = inputs(8300 + N + W, (B, H, N, 64), dtype, with_dout=True)
    ad = dev_alpha(a)
    o, lse = F.fwd_dev(q, k, v, W, ad, rng, base, 10000.0, mode)
    dq, dk, dv, da = F.bwd_dev(q, k, v, o, lse, do, W, ad, rng, base, 10000.0, mode)
    torch.cuda.synchronize()
    rq, rk, rv, ra, rsc = O.backward(q64, k64, v64, d64, W, a, base, 10000.0, mode, workers=WORKERS,
                                     return_scale=True)
    eq, ek, ev = grad_excess(host(dq), rq, dtype), grad_excess(host(dk), rk, dtype), grad_excess(host(dv), rv, dtype)
    got_a = float(da.item())
    say(f"  dQ {eq:.2e} dK {ek:.2e} dV {ev:.2e}")
    assert max(eq, ek, ev) <= TOL[dtype]
    if mode == INT:
        assert got_a == 0.0
    else:
        dalpha_check(got_a, ra, rsc, dtype)


DEC = [
    (2, 4, 3000, 12, 1.37, LEARNED, FIB_BASE, BF16),
    (1, 8, 4096, 12, 1.0, (1.0, 1.0), FIB_BASE, BF16),
    (1, 2, 300, 130, 1.0, (0.5, 2.0), FIB_BASE, BF16),
    (2, 3, 1000, 12, 1.21, LEARNED, FIB_BASE, F32),
    (1, 1, 1, 12, 1.0, LEARNED, FIB_BASE, BF16),
]


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("case", DEC, ids=[fwd_ids(c) for c in DEC])
def test_decode_device_alpha(case, mode):
    B, H, N, W, alpha, rng, base, dtype = case
    a = np.float32(alpha)
    say("decode_dev", fwd_ids(case), "mode", mode)
    (q, q64), (k, k64), (v, v64) = inputs(8500 + N + W, (B, H, N, 64), dtype)
    qd = q[:, :, N - 1, :].contiguous()
    o, lse = F.decode_dev(qd, k, v, W, dev_alpha(a), rng, base, 10000.0, mode)
    oh, lh = F.decode(qd, k, v, W, a, base, 10000.0, mode)
    torch.cuda.synchronize()
    # one kernel, the same table: the host-alpha call's result exactly
    assert torch.equal(o, oh) and torch.equal(lse, lh)
    go, gl = host(o), host(lse)
    eo = el = 0.0
    for b in range(B):
        for h in range(H):
            ro, rl = O.forward_rows(q64[b, h], k64[b, h], v64[b, h], np.array([N - 1]), W, a, base, 10000.0, mode)
            eo = max(eo, maxabs(go[b, h], ro[0]))
            el = max(el, maxabs(gl[b, h], rl[0]))
    say(f"  vs oracle O {eo:.3e} LSE {el:.3e}")
    assert eo <= TOL[dtype] and el <= TOL[dtype]


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("alpha", [0.2, 1.9, float("nan")], ids=["below", "above", "nan"])
def test_alpha_is_clamped_into_range(alpha, mode):
    """alpha outside [lo, hi] gives the result at the nearest end (NaN: the low end)."""
    rng = LEARNED
    ac = np.float32(rng[0]) if np.isnan(alpha) else clamp(alpha, rng)
    say("clamp", alpha, "->", ac, "mode", mode)
    (q, _), (k, _), (v, _), (do, _) = inputs(8700, (1, 2, 2500, 64), BF16, with_dout=True)
    ad = dev_alpha(alpha)
    o, lse = F.fwd_dev(q, k, v, 12, ad, rng, FIB_BASE, 10000.0, mode)
    oh, lh = F.fwd(q, k, v, 12, ac, FIB_BASE, 10000.0, mode)
    dq, dk, dv, _ = F.bwd_dev(q, k, v, o, lse, do, 12, ad, rng, FIB_BASE, 10000.0, mode)
    dqh, dkh, dvh, _ = F.bwd(q, k, v, oh, lh, do, 12, ac, FIB_BASE, 10000.0, mode)
    qd = q[:, :, -1, :].contiguous()
    od, _ = F.decode_dev(qd, k, v, 12, ad, rng, FIB_BASE, 10000.0, mode)
    odh, _ = F.decode(qd, k, v, 12, ac, FIB_BASE, 10000.0, mode)
    torch.cuda.synchronize()
    e = max(maxabs(host(o), host(oh)), maxabs(host(lse), host(lh)))
    g = max(grad_excess(host(dq), host(dqh), BF16), grad_excess(host(dk), host(dkh), BF16),
            grad_excess(host(dv), host(dvh), BF16))
    say(f"  fwd diff {e:.3e} grad excess {g:.3e}")
    assert e <= TOL[BF16] and g <= TOL[BF16]
    assert torch.equal(od, odh)


def test_device_alpha_reads_alpha_at_run_time():
    """The plan is rebuilt from device memory on every call: changing alpha in place between
    calls (no new host value) changes the result accordingly."""
    (q, _), (k, _), (v, _) = inputs(8800, (1, 2, 2000, 64), BF16)
    ad = dev_alpha(0.8)
    plan = torch.empty(F.plan_bytes(), dtype=torch.uint8, device="cuda")
    o1, _ = F.fwd_dev(q, k, v, 12, ad, LEARNED, FIB_BASE, 10000.0, INTERP, plan=plan)
    o1 = o1.clone()
    ad.fill_(1.3)
    o2, _ = F.fwd_dev(q, k, v, 12, ad, LEARNED, FIB_BASE, 10000.0, INTERP, plan=plan)
    h1, _ = F.fwd(q, k, v, 12, np.float32(0.8), FIB_BASE, 10000.0, INTERP)
    h2, _ = F.fwd(q, k, v, 12, np.float32(1.3), FIB_BASE, 10000.0, INTERP)
    torch.cuda.synchronize()
    d1, d2 = maxabs(host(o1), host(h1)), maxabs(host(o2), host(h2))
    say(f"in-place alpha change: {d1:.3e} {d2:.3e}")
    assert d1 <= TOL[BF16] and d2 <= TOL[BF16]
    assert maxabs(host(o1), host(o2)) > 10 * TOL[BF16]


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_autograd_device_alpha_path(mode):
    """fib_sparse_attention with alpha_range: the device-alpha entry points' results exactly."""
    (q, _), (k, _), (v, _), (do, _) = inputs(8900, (2, 2, 1500, 64), BF16, with_dout=True)
    alpha = torch.tensor([1.11], dtype=torch.float32, device="cuda", requires_grad=True)
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = fib_sparse_attention(qq, kk, vv, alpha, 12, FIB_BASE, 10000.0, mode, alpha_range=LEARNED)
    (o.float() * do.float()).sum().backward()
    ad = dev_alpha(1.11)
    of, lf = F.fwd_dev(q, k, v, 12, ad, LEARNED, FIB_BASE, 10000.0, mode)
    dq, dk, dv, da = F.bwd_dev(q, k, v, of, lf, do, 12, ad, LEARNED, FIB_BASE, 10000.0, mode)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), of)
    assert torch.equal(qq.grad, dq) and torch.equal(kk.grad, dk) and torch.equal(vv.grad, dv)
    assert float(alpha.grad.item()) == float(da.item())


# Layout of one plan (the library's internal DevPlan): the table {int n; int dist[32];
# float w[32]; float f[32]} and two ring splits {int n_cov, n_far, need, early_rows; int
# dist[16]; float w[16], f[16]; int far_dist[4]; float far_w[4], far_f[4]; int unc_dist[8]}
# for 8- and 4-wave kernels.
PLAN_WORDS = 97 + 2 * 72


def decode_plan(words):
    n = int(words[0])
    dist = words[1:33].astype(np.int32)
    w = words[33:65].view(np.float32)
    f = words[65:97].view(np.float32)
    splits = []
    for s0 in (97, 97 + 72):
        sw = words[s0:s0 + 72]
        splits.append(dict(n_cov=int(sw[0]), n_far=int(sw[1]), need=int(sw[2]), early_rows=int(sw[3]),
                           dist=sw[4:20].astype(np.int32), far_dist=sw[52:56].astype(np.int32)))
    return n, dist, w, f, splits


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("W,base,N", [(12, FIB_BASE, 4096), (1, FIB_BASE, 131072), (40, POW2_BASE, 3000),
                                      (3, (1, 2, 3, 4, 5, 6, 7, 8), 100),
                                      (12, (1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 511, 512, 610), 900)],
                         ids=["fib-W12", "fib-W1", "pow2-W40", "dense-base", "near-dup"])
def test_device_built_tables_equal_host_and_oracle_tables(W, base, N, mode):
    """The plans the device builds (one per layer of a 256-layer call) hold exactly the host
    table and the oracle's offsets, and the ring splits follow the table."""
    assert F.plan_bytes() == 4 * PLAN_WORDS
    L = 256
    al = random_alpha_grid(9900 + W + N, L, 0.3, 3.0)
    al[:4] = [0.5, 1.0, 1.5, 2.0 / 3.0]  # exact halves: rounding ties
    plan = torch.empty(F.layers_plan_bytes(L), dtype=torch.uint8, device="cuda")
    # only the plans are inspected (the splits depend on N)
    kk = torch.zeros((L, 1, 1, N, 64), dtype=torch.bfloat16, device="cuda")
    F.fwd_layers(kk, kk, kk, W, torch.from_numpy(al).cuda(), base, 10000.0, mode, alpha_range=(0.3, 3.0), plan=plan,
                 with_lse=False)
    torch.cuda.synchronize()
    words = plan.cpu().numpy().view(np.uint32).reshape(L, PLAN_WORDS)
    for l in range(L):
        n, dist, w, f, splits = decode_plan(words[l])
        hd, hw, hf = F.offset_table(al[l], base, W, mode)
        assert n == len(hd), (l, al[l])
        assert list(dist[:n]) == hd and np.array_equal(w[:n], np.array(hw, dtype=np.float32))
        if mode == INTERP:
            assert list(f[:n].astype(np.int64)) == hf
            od = [c for _, c, _ in O.interp_entries(al[l], base, W)]
        else:
            od = O.int_offsets(al[l], base, W)
        assert list(dist[:n]) == [int(x) for x in od]
        usable = sum(1 for x in hd if x < N)
        for sp, waves in zip(splits, (8, 4)):
            reach = 512 - 16 * waves
            cov = sum(1 for x in hd[:usable] if x <= reach)
            assert sp["n_cov"] == cov and sp["n_far"] == usable - cov
            assert sp["need"] == max([16] + hd[:cov]) and sp["early_rows"] == max([16] + hd[:usable])
            assert list(sp["dist"][:cov]) == hd[:cov]
            far = hd[cov:usable][:4]
            assert list(sp["far_dist"][:len(far)]) == far
