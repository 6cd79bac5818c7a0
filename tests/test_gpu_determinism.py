"""Outputs are a function of the inputs alone: repeated calls give bitwise-identical results.

Each case runs the forward and the backward three times. Between the runs the memory the
calls write or may read is refilled with different patterns: the caller's output and
workspace buffers (NaN bits, zeros, random bytes), and freed blocks of the caching
allocator that the binding's own allocations reuse. A kernel that reads a word before
writing it, races within a workgroup, or depends on the timing of other waves shows up here
as a difference between runs, including in dalpha, which sums many per-query parts that
nearly cancel and so amplifies any such error.

The cases cover the kernel families that the launch logic picks: the LDS-ring kernels at
8 and 4 waves with 8 and 16 covered slots and up to 4 far slots, far rows read pre-rotated,
the general kernels (fp32, window wider than the band), the gather kernel of small forwards,
alpha in device memory, and layer stacks.
"""
import numpy as np
import pytest
import torch

import fibonacci_offset_dilated_amd as F
from fibonacci_offset_dilated_amd.workloads import BF16, F32, FIB_BASE, INT, INTERP, POW2_BASE
from gpu_util import say

pytestmark = pytest.mark.gpu

FILLS = ("nan", "zero", "random")

CASES = [
    # (name, (B, H, N), W, alpha, base, dtype)
    ("ring-nc16-nf3-w1", (2, 1, 4100), 1, 1.5, POW2_BASE, BF16),
    ("ring-nc16-nf4-4waves", (1, 2, 8192), 1, 1.5, POW2_BASE + (4096,), BF16),
    ("ring-fib-long", (1, 4, 16384), 12, 1.5, FIB_BASE, BF16),
    ("ring-nc8", (1, 2, 3000), 12, 0.6, FIB_BASE, BF16),
    ("ring-mixed-far", (1, 3, 5000), 16, 1.0, (1, 2, 512, 513, 700), BF16),
    ("small-8x8x1024", (8, 8, 1024), 12, 1.5, FIB_BASE, BF16),
    ("gather-f32", (1, 1, 1024), 12, 1.5, FIB_BASE, F32),
    ("general-f32", (1, 2, 40000), 12, 1.5, FIB_BASE, F32),
    ("wide-window", (1, 2, 2048), 40, 1.0, FIB_BASE, BF16),
    ("wide-window-large", (1, 2, 40000), 40, 1.0, FIB_BASE, BF16),
    # interpolated: far K rows read as the rotated rows the query side wrote (segments of 2048
    # rows whose workgroups first rotate the rows before them, which the previous segment's
    # workgroup also writes)
    ("ring-rotated-far", (1, 16, 65536), 12, 0.9, FIB_BASE, BF16),
]


def fill_(t: torch.Tensor, how: str, gen: torch.Generator) -> torch.Tensor:
    b = t.view(torch.uint8)
    if how == "nan":
        b.fill_(0xFF)
    elif how == "zero":
        b.zero_()
    else:
        b.copy_(torch.randint(0, 256, b.shape, dtype=torch.uint8, device=b.device, generator=gen))
    return t


def churn(how: str, gen: torch.Generator, nbytes: int) -> None:
    """Leaves freed blocks holding the pattern for the binding's own allocations to reuse."""
    junk = [fill_(torch.empty(max(16, nbytes >> s), dtype=torch.uint8, device="cuda"), how, gen) for s in range(0, 6)]
    torch.cuda.synchronize()
    del junk


def rand_inputs(seed, shape, dtype, n):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dt = torch.bfloat16 if dtype == BF16 else torch.float32
    return [torch.randn(shape, generator=g, device="cuda").to(dt) for _ in range(n)]


def same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def run_single(case, mode, how, gen):
    name, (B, H, N), W, alpha, base, dtype = case
    alpha = np.float32(alpha)
    q, k, v, do = rand_inputs(sum(map(ord, name)), (B, H, N, 64), dtype, 4)
    o = fill_(torch.empty_like(q), how, gen)
    lse = fill_(torch.empty((B, H, N), dtype=torch.float32, device="cuda"), how, gen)
    F.fwd(q, k, v, W, alpha, base, 10000.0, mode, out=o, lse=lse)
    need = F.bwd_workspace_size(B, H, N, 64, dtype, mode, W, alpha, base)
    ws = fill_(torch.empty(max(need, 16), dtype=torch.uint8, device="cuda"), how, gen)
    dq, dk, dv = (fill_(torch.empty_like(q), how, gen) for _ in range(3))
    da = fill_(torch.empty(1, dtype=torch.float32, device="cuda"), how, gen)
    F.bwd(q, k, v, o, lse, do, W, alpha, base, 10000.0, mode, dq=dq, dk=dk, dv=dv, dalpha=da, workspace=ws)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dalpha": da}


def check_runs(label, runs):
    ref = runs[0]
    for r, got in enumerate(runs[1:], start=1):
        bad = [key for key in ref if not same(ref[key], got[key])]
        if "dalpha" in ref:
            say(f"  {label} run {r}: dalpha {float(got['dalpha'][0]):.9g} (run 0: {float(ref['dalpha'][0]):.9g})")
        assert not bad, (label, r, bad)


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_repeated_calls_bitwise(case, mode):
    say("determinism", case[0], "mode", mode)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    runs = []
    for how in FILLS:
        churn(how, gen, 64 << 20)
        runs.append(run_single(case, mode, how, gen))
    check_runs(case[0], runs)


@pytest.mark.parametrize("shape", [(1, 4, 16384, 1.37, (1.0, 1.5)), (1, 16, 131072, 0.9, (0.85, 0.95))],
                         ids=["h4", "rotated-far"])
@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_repeated_calls_bitwise_device_alpha(mode, shape):
    B, H, N, a, rng = shape
    W = 12
    say("determinism device alpha", B, H, N, W, a, rng, mode)
    q, k, v, do = rand_inputs(5, (B, H, N, 64), BF16, 4)
    alpha = torch.tensor([a], dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    runs = []
    for how in FILLS:
        churn(how, gen, 64 << 20)
        o, lse = F.fwd_dev(q, k, v, W, alpha, rng, FIB_BASE, 10000.0, mode)
        dq, dk, dv, da = F.bwd_dev(q, k, v, o, lse, do, W, alpha, rng, FIB_BASE, 10000.0, mode)
        torch.cuda.synchronize()
        runs.append({"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dalpha": da})
    check_runs("device alpha", runs)


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_repeated_calls_bitwise_layers(mode):
    L, B, H, N, W = 4, 1, 2, 2048, 12
    say("determinism layers", L, B, H, N, W, mode)
    q, k, v, do = rand_inputs(6, (L, B, H, N, 64), BF16, 4)
    alphas = np.array([F.schedule_alpha(F.SCHED_LINEAR, l, L) for l in range(L)], dtype=np.float32)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    runs = []
    for how in FILLS:
        churn(how, gen, 64 << 20)
        o, lse = F.fwd_layers(q, k, v, W, alphas, FIB_BASE, 10000.0, mode)
        dq, dk, dv, da = F.bwd_layers(q, k, v, o, lse, do, W, alphas, FIB_BASE, 10000.0, mode)
        torch.cuda.synchronize()
        runs.append({"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dalpha": da})
    check_runs("layers", runs)
