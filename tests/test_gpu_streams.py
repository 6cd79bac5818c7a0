"""Stream semantics of the C ABI, through the Python binding.

The calls enqueue their kernels on the caller's stream and return without synchronizing:
work on a side stream (current-stream context or the explicit `stream` argument) gives the
same bits as on the default stream, and a forward + backward captured in a HIP graph
replays correctly with new inputs written in place between replays (and eager work in
between), including the device-alpha calls with alpha updated in device memory. Every
kernel here is deterministic, so the comparisons are bitwise.
"""
import numpy as np
import pytest
import torch

import fibonacci_offset_dilated_amd as F
from fibonacci_offset_dilated_amd.workloads import BF16, FIB_BASE, INT, INTERP
from gpu_util import inputs, say

pytestmark = pytest.mark.gpu

B, H, N, W = 1, 2, 1500, 12
ALPHA = np.float32(1.37)


def _buffers(q, mode):
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dal = torch.empty(1, dtype=torch.float32, device=q.device)
    ws = torch.empty(F.bwd_workspace_size(B, H, N, 64, F.BF16, mode), dtype=torch.uint8, device=q.device)
    return o, lse, dq, dk, dv, dal, ws


def _step(q, k, v, do, mode, bufs, stream=None):
    o, lse, dq, dk, dv, dal, ws = bufs
    F.fwd(q, k, v, W, ALPHA, FIB_BASE, 10000.0, mode, out=o, lse=lse, stream=stream)
    F.bwd(q, k, v, o, lse, do, W, ALPHA, FIB_BASE, 10000.0, mode, dq=dq, dk=dk, dv=dv, dalpha=dal, workspace=ws,
          stream=stream)


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_side_stream_matches_default_stream(mode):
    say("side stream", mode)
    (q, _), (k, _), (v, _), (do, _) = inputs(4401, (B, H, N, 64), BF16, with_dout=True)
    ref = _buffers(q, mode)
    _step(q, k, v, do, mode, ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    got = _buffers(q, mode)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # the binding picks up the current stream
        _step(q, k, v, do, mode, got)
    side.synchronize()
    assert _same(got[:6], ref[:6])
    got2 = _buffers(q, mode)
    side.wait_stream(torch.cuda.current_stream())
    _step(q, k, v, do, mode, got2, stream=side)  # explicit stream argument
    side.synchronize()
    assert _same(got2[:6], ref[:6])


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_graph_capture_replays(mode):
    say("graph capture", mode)
    sets = [inputs(4500 + s, (B, H, N, 64), BF16, with_dout=True) for s in range(3)]
    dev = [[t for t, _ in s] for s in sets]
    # eager references, one per input set
    refs = []
    for q, k, v, do in dev:
        bufs = _buffers(q, mode)
        _step(q, k, v, do, mode, bufs)
        refs.append(bufs)
    torch.cuda.synchronize()
    # static inputs and outputs for the graph
    sq, sk, sv, sd = (t.clone() for t in dev[0])
    gb = _buffers(sq, mode)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(sq, sk, sv, sd, mode, gb)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(sq, sk, sv, sd, mode, gb)
    for rep in range(4):
        s = rep % 3
        for dst, src in zip((sq, sk, sv, sd), dev[s]):
            dst.copy_(src)
        g.replay()
        # eager work between replays, on the same stream
        scratch = _buffers(sq, mode)
        _step(dev[(s + 1) % 3][0], dev[(s + 1) % 3][1], dev[(s + 1) % 3][2], dev[(s + 1) % 3][3], mode, scratch)
        torch.cuda.synchronize()
        assert _same(gb[:6], refs[s][:6]), f"replay {rep} (input set {s})"
        assert _same(scratch[:6], refs[(s + 1) % 3][:6])


def test_graph_capture_device_alpha_updates():
    """The learned schedule's step: alpha lives in device memory, so a captured forward +
    backward follows updates written into it between replays."""
    say("graph capture, device alpha")
    mode, rng = INTERP, (0.5, 1.5)
    (q, _), (k, _), (v, _), (do, _) = inputs(4601, (B, H, N, 64), BF16, with_dout=True)
    alphas = [np.float32(1.04), np.float32(0.93), np.float32(1.21)]
    plan = torch.empty(F.plan_bytes(), dtype=torch.uint8, device=q.device)

    def step(a_dev, bufs):
        o, lse, dq, dk, dv, dal, ws = bufs
        F.fwd_dev(q, k, v, W, a_dev, rng, FIB_BASE, 10000.0, mode, out=o, lse=lse, plan=plan)
        F.bwd_dev(q, k, v, o, lse, do, W, a_dev, rng, FIB_BASE, 10000.0, mode, dq=dq, dk=dk, dv=dv, dalpha=dal,
                  workspace=ws, plan=plan)

    refs = []
    for a in alphas:
        bufs = _buffers(q, mode)
        step(torch.tensor([a], dtype=torch.float32, device=q.device), bufs)
        torch.cuda.synchronize()
        refs.append(bufs)
    a_static = torch.tensor([alphas[0]], dtype=torch.float32, device=q.device)
    gb = _buffers(q, mode)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(a_static, gb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(a_static, gb)
    for rep in range(5):
        s = rep % 3
        a_static.fill_(float(alphas[s]))
        g.replay()
        torch.cuda.synchronize()
        assert _same(gb[:6], refs[s][:6]), f"replay {rep} (alpha {alphas[s]})"


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_explicit_stream_binding_allocations(mode):
    """Explicit `stream` argument with every buffer left to the binding (outputs, backward
    workspace, device-alpha plan): while the side stream's kernels may still run, the default
    stream allocates and overwrites memory of the same sizes. The binding allocates on the
    side stream, so those blocks are not handed out again before the side stream's work
    ends, and the results equal a default-stream call bit for bit."""
    say("explicit stream, binding-allocated buffers", mode)
    (q, _), (k, _), (v, _), (do, _) = inputs(4601, (B, H, N, 64), BF16, with_dout=True)
    ref_o, ref_lse = F.fwd(q, k, v, W, ALPHA, FIB_BASE, 10000.0, mode)
    ref_g = F.bwd(q, k, v, ref_o, ref_lse, do, W, ALPHA, FIB_BASE, 10000.0, mode)
    a_dev = torch.tensor([ALPHA], dtype=torch.float32, device=q.device)
    ref_dev = F.fwd_dev(q, k, v, W, a_dev, (0.5, 1.5), FIB_BASE, 10000.0, mode)
    ref_gdev = F.bwd_dev(q, k, v, ref_dev[0], ref_dev[1], do, W, a_dev, (0.5, 1.5), FIB_BASE, 10000.0, mode)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    ws_bytes = F.bwd_workspace_size(B, H, N, 64, F.BF16, mode)
    for rep in range(3):
        side.wait_stream(torch.cuda.current_stream())
        o, lse = F.fwd(q, k, v, W, ALPHA, FIB_BASE, 10000.0, mode, stream=side)
        g = F.bwd(q, k, v, o, lse, do, W, ALPHA, FIB_BASE, 10000.0, mode, stream=side)
        od, ld = F.fwd_dev(q, k, v, W, a_dev, (0.5, 1.5), FIB_BASE, 10000.0, mode, stream=side)
        gd = F.bwd_dev(q, k, v, od, ld, do, W, a_dev, (0.5, 1.5), FIB_BASE, 10000.0, mode, stream=side)
        # the default stream grabs and scribbles over memory of the sizes just released
        junk = [torch.full((max(ws_bytes, 16),), 0xAB, dtype=torch.uint8, device=q.device),
                torch.full((F.plan_bytes(),), 0xCD, dtype=torch.uint8, device=q.device),
                torch.full_like(q, float("nan")), torch.full_like(ref_lse, float("nan"))]
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse), rep
        assert _same(g[:3], ref_g[:3]) and (mode == INT or torch.equal(g[3], ref_g[3])), rep
        assert torch.equal(od, ref_dev[0]) and _same(gd[:3], ref_gdev[:3]), rep
        del junk
