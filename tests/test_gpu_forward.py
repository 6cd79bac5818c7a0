"""GPU parity of the forward pass against the CPU oracle, through the C ABI.

Values: max-abs error on O and LSE within 1e-4 (fp32 inputs) / 2e-2 (bf16 inputs).
Index sets: the library's device export equals the oracle's, bit for bit.
Workloads: the five measured configurations (full comparison where the oracle is quick,
sampled heads or rows at the large ones), plus ragged and degenerate shapes.
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
from gpu_util import TOL, host, inputs, maxabs, say

pytestmark = pytest.mark.gpu
WORKERS = min(16, len(os.sched_getaffinity(0)))


def alpha_of(w, layer):
    if w.schedule == "fixed1":
        return F.schedule_alpha(F.SCHED_FIXED, layer, 16)
    if w.schedule == "linear":
        return F.schedule_alpha(F.SCHED_LINEAR, layer, 16)
    if w.schedule == "coprime":
        return F.schedule_alpha(F.SCHED_COPRIME, layer, 16)
    if w.schedule == "layer15_linear":
        return F.schedule_alpha(F.SCHED_LINEAR, 15, 16)
    return uniform_alphas(UNIFORM_ALPHA_SEED, 16, *UNIFORM_ALPHA_RANGE)[layer]


def run_fwd(qkv, W, alpha, base, mode):
    (q, _), (k, _), (v, _) = qkv[:3]
    o, lse = F.fwd(q, k, v, W, alpha, base, 10000.0, mode)
    torch.cuda.synchronize()
    return o, lse


def check_full(qkv, W, alpha, base, mode, dtype, heads=None):
    (_, q64), (_, k64), (_, v64) = qkv[:3]
    o, lse = run_fwd(qkv, W, alpha, base, mode)
    oh, lh = host(o), host(lse)
    if heads is None:
        ro, rl = O.forward(q64, k64, v64, W, alpha, base, 10000.0, mode, workers=WORKERS)
        eo, el = maxabs(oh, ro), maxabs(lh, rl)
    else:
        eo = el = 0.0
        for b, h in heads:
            ro, rl = O.forward(q64[b:b + 1, h:h + 1], k64[b:b + 1, h:h + 1], v64[b:b + 1, h:h + 1], W, alpha, base,
                               10000.0, mode)
            eo = max(eo, maxabs(oh[b, h], ro[0, 0]))
            el = max(el, maxabs(lh[b, h], rl[0, 0]))
    assert np.isfinite(oh).all()
    assert eo <= TOL[dtype] and el <= TOL[dtype], (eo, el)
    return eo, el


def check_index_set(N, W, alpha, base, mode):
    got = F.index_set(N, W, alpha, base, mode).cpu().numpy()
    want = O.index_sets(N, W, alpha, base, mode)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


# ---- the five workloads ----------------------------------------------------------------

def test_single_head_fp32():
    w = BY_CONFIG[1]
    say("single head fp32 N=1024 W=12 alpha=1 INT")
    qkv = inputs(seed_for(1, 0, 12, 0), (w.B, w.H, w.N, w.D), F32)
    a = alpha_of(w, 0)
    eo, el = check_full(qkv, 12, a, FIB_BASE, INT, F32)
    check_index_set(w.N, 12, a, FIB_BASE, INT)
    say("  max err O", eo, "LSE", el)


@pytest.mark.parametrize("W", [6, 8, 10, 12])
@pytest.mark.parametrize("layer", range(16))
def test_staggered_linear_layers(W, layer):
    w = BY_CONFIG[2]
    a = alpha_of(w, layer)
    say(f"staggered linear B8H8N1024 bf16 W={W} layer={layer} alpha={a}")
    qkv = inputs(seed_for(2, 0, W, layer), (w.B, w.H, w.N, w.D), BF16)
    check_full(qkv, W, a, FIB_BASE, INT, BF16)
    check_index_set(w.N, W, a, FIB_BASE, INT)


@pytest.mark.parametrize("layer", range(16))
def test_learned_dilation_layers_forward(layer):
    w = BY_CONFIG[3]
    a = alpha_of(w, layer)
    say(f"learned dilation B8H8N1024 bf16 INTERP W=12 layer={layer} alpha={a}")
    qkv = inputs(seed_for(3, 0, 12, layer), (w.B, w.H, w.N, w.D), BF16)
    check_full(qkv, 12, a, FIB_BASE, INTERP, BF16)
    check_index_set(w.N, 12, a, FIB_BASE, INTERP)


@pytest.mark.parametrize("base_id,base", [(0, FIB_BASE), (1, POW2_BASE)], ids=["fib", "pow2"])
@pytest.mark.parametrize("layer", range(16))
def test_coprime_extrapolation_layers(base_id, base, layer):
    w = BY_CONFIG[4]
    a = alpha_of(w, layer)
    say(f"coprime B4H8N4096 bf16 W=12 base={base_id} layer={layer} alpha={a}")
    qkv = inputs(seed_for(4, base_id, 12, layer), (w.B, w.H, w.N, w.D), BF16)
    heads = [((layer + 3 * base_id) % 4, (layer * 5) % 8), ((layer + 1) % 4, (layer * 3 + 1) % 8)]
    check_full(qkv, 12, a, base, INT, BF16, heads=heads)
    check_index_set(w.N, 12, a, base, INT)


@pytest.fixture(scope="module")
def long_inputs():
    w = BY_CONFIG[5]
    say("long context inputs B1H32N131072 bf16")
    return inputs(seed_for(5, 0, 12, 15), (w.B, w.H, w.N, w.D), BF16)


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_long_context_sampled_rows(long_inputs, mode):
    w = BY_CONFIG[5]
    a = alpha_of(w, 15)
    say(f"long context N=131072 H=32 alpha={a} mode={mode}")
    o, lse = run_fwd(long_inputs, 12, a, FIB_BASE, mode)
    (_, q64), (_, k64), (_, v64) = long_inputs[:3]
    o_h, lse_h = host(o[0]), host(lse[0])
    eo = el = 0.0
    # every head: the sequence start, the rows where the far entries start (980..1500), the
    # end, and random rows; four heads with a denser random sample
    for h in range(w.H):
        rng = np.random.default_rng(100 * h + mode)
        n_rand = 600 if h in (0, 7, 19, 31) else 150
        rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(980, 1500, 1 if h in (0, 31) else 7),
                                         rng.integers(0, w.N, n_rand), np.arange(w.N - 70, w.N)]))
        ro, rl = O.forward_rows(q64[0, h], k64[0, h], v64[0, h], rows, 12, a, FIB_BASE, 10000.0, mode)
        eo = max(eo, maxabs(o_h[h][rows], ro))
        el = max(el, maxabs(lse_h[h][rows], rl))
    say("  max err O", eo, "LSE", el, "over all", w.H, "heads")
    assert eo <= TOL[BF16] and el <= TOL[BF16]
    assert torch.isfinite(o.float()).all().item()
    check_index_set(w.N, 12, a, FIB_BASE, mode)


# ---- edge cases ------------------------------------------------------------------------

EDGE = [
    # (B, H, N, W, alpha, base)
    (1, 1, 1, 1, 1.0, FIB_BASE),
    (1, 2, 2, 12, 1.0, FIB_BASE),
    (2, 3, 3, 1, 0.5, FIB_BASE),
    (1, 2, 63, 12, 1.5, FIB_BASE),
    (1, 2, 65, 6, 0.7, FIB_BASE),
    (2, 1, 200, 16, 1.3, FIB_BASE),
    (1, 1, 300, 17, 1.1, FIB_BASE),
    (1, 1, 257, 40, 0.9, POW2_BASE),
    (1, 2, 130, 130, 1.0, FIB_BASE),      # window covers the sequence: causal attention
    (1, 1, 100, 12, 40.0, FIB_BASE),      # every offset beyond the sequence
    (1, 1, 1000, 1, 1.0, (1,)),            # one offset of 1 next to a window of 1
    (1, 1, 777, 12, 0.5, tuple(range(1, 33))),
]


@pytest.mark.parametrize("dtype", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("case", EDGE, ids=[f"B{c[0]}H{c[1]}N{c[2]}W{c[3]}a{c[4]}" for c in EDGE])
def test_edge_shapes(case, mode, dtype):
    B, H, N, W, alpha, base = case
    say("edge", case, mode, dtype)
    qkv = inputs(1000 + N + W, (B, H, N, 64), dtype)
    check_full(qkv, W, np.float32(alpha), base, mode, dtype)
    check_index_set(N, W, np.float32(alpha), base, mode)


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_probes_ones_and_zero_query(mode):
    N, W, a = 1500, 12, np.float32(1.37)
    say("probes", mode)
    (q, _), (k, k64), (v, _) = inputs(77, (1, 2, N, 64), BF16)
    ones = torch.ones_like(v)
    o, _ = F.fwd(q, k, ones, W, a, FIB_BASE, 10000.0, mode)
    assert maxabs(host(o), 1.0) <= 1e-6
    _, lse = F.fwd(torch.zeros_like(q), k, v, W, a, FIB_BASE, 10000.0, mode)
    ids = O.index_sets(N, W, a, FIB_BASE, mode)
    n = (ids >= 0).sum(axis=1)
    assert maxabs(host(lse)[0, 0], np.log(n)) <= 1e-5


@pytest.mark.parametrize("dtype", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_nan_locality(mode, dtype):
    """A NaN in one K or V row reaches every query that reads the row. A K row reaches no
    other query on either kernel: logits outside a query's attended set are selected away,
    not offset. For V rows the general kernel (fp32 here) touches nothing else either; the
    MFMA kernel (bf16) multiplies whole 16-row V blocks by weights that are 0 for unattended
    rows, and 0 * NaN = NaN, so there the check is that NaN stays within the queries whose
    blocks cover the row."""
    N, W, a = 1700, 12, np.float32(1.37) if mode == INTERP else np.float32(1.3)
    say("nan locality", mode, dtype)
    (q, _), (k, _), (v, _) = inputs(78, (1, 1, N, 64), dtype)
    ids = O.index_sets(N, W, a, FIB_BASE, mode)
    reach = int(ids.shape[1] and max(0, np.max(np.arange(N)[:, None] - np.where(ids >= 0, ids, np.arange(N)[:, None]))))
    for tensor_name, j0 in (("k", 333), ("v", 1000)):
        kk, vv = k.clone(), v.clone()
        (kk if tensor_name == "k" else vv)[0, 0, j0, 5] = float("nan")
        o, _ = F.fwd(q, kk, vv, W, a, FIB_BASE, 10000.0, mode)
        bad = torch.isnan(o[0, 0]).any(dim=1).cpu().numpy()
        reads = (ids == j0).any(axis=1)
        if mode == INTERP:
            hi = np.where(ids[:, W:] >= 0, ids[:, W:] + 1, -1)
            reads |= (hi == j0).any(axis=1)
        assert not (reads & ~bad).any(), tensor_name
        if dtype == F32 or tensor_name == "k":
            assert np.array_equal(bad, reads), tensor_name
        else:
            near = np.zeros(N, dtype=bool)
            near[max(0, j0 - 16):min(N, j0 + reach + 32)] = True
            assert not (bad & ~near).any(), tensor_name


def test_deterministic_repeat():
    say("determinism")
    qkv = inputs(5, (2, 4, 3000, 64), BF16)
    for mode in (INT, INTERP):
        o1, l1 = run_fwd(qkv, 12, np.float32(1.5), FIB_BASE, mode)
        o2, l2 = run_fwd(qkv, 12, np.float32(1.5), FIB_BASE, mode)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---- cases aimed at the ring kernel (bf16, W <= 16): segment edges, ring reach, far rows ----

RING = [
    # (B, H, N, W, alpha, base)
    (1, 1, 10000, 12, 1.5, FIB_BASE),          # many short segments, far entries 566/915/1480
    (1, 3, 5000, 16, 1.0, (1, 2, 512, 513, 700)),  # distances 512 (ring) and 513 (global)
    (2, 1, 4100, 1, 1.5, POW2_BASE),           # W = 1, far rows up to 3072
    (1, 2, 70, 6, 0.5, FIB_BASE),              # one partial step
    (1, 1, 1, 12, 1.0, FIB_BASE),
    (3, 5, 1500, 10, 1.3, FIB_BASE),
    (1, 1, 2000, 12, 1.0001, (1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 511, 512, 610)),
]


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("case", RING, ids=[f"B{c[0]}H{c[1]}N{c[2]}W{c[3]}a{c[4]}n{len(c[5])}" for c in RING])
def test_ring_cases(case, mode):
    B, H, N, W, alpha, base = case
    say("ring", case, mode)
    qkv = inputs(3000 + N + W, (B, H, N, 64), BF16)
    check_full(qkv, W, np.float32(alpha), base, mode, BF16)


# ---- long sequences with many heads: many segments per head, ragged last segment, head counts
# that are not a multiple of 8

LONG_MANY = [
    # (B, H, N, W, alpha, base, heads checked)
    (2, 16, 33000, 12, 1.5, FIB_BASE, [(0, 0), (0, 9), (1, 15)]),   # ragged last segment
    (1, 13, 81000, 12, 1.0, FIB_BASE, [(0, 0), (0, 6), (0, 12)]),   # heads not a multiple of 8
]


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("case", LONG_MANY, ids=[f"B{c[0]}H{c[1]}N{c[2]}a{c[4]}" for c in LONG_MANY])
def test_long_many_heads(case, mode):
    B, H, N, W, alpha, base, heads = case
    alpha = np.float32(alpha)
    say("long many heads", case[:5], mode)
    qkv = inputs(4000 + N + H, (B, H, N, 64), BF16)
    o, lse = run_fwd(qkv, W, alpha, base, mode)
    rng = np.random.default_rng(N)
    edges = np.concatenate([np.arange(k * 512 - 3, k * 512 + 3) for k in range(1, 12)])
    rows = np.unique(np.concatenate([np.arange(0, 40), edges, rng.integers(0, N, 300), np.arange(N - 40, N)]))
    (_, q64), (_, k64), (_, v64) = qkv[:3]
    eo = el = 0.0
    for b, h in heads:
        ro, rl = O.forward_rows(q64[b, h], k64[b, h], v64[b, h], rows, W, alpha, base, 10000.0, mode)
        eo = max(eo, maxabs(host(o[b, h])[rows], ro))
        el = max(el, maxabs(host(lse[b, h])[rows], rl))
    say("  max err O", eo, "LSE", el)
    assert eo <= TOL[BF16] and el <= TOL[BF16]
    assert torch.isfinite(o.float()).all().item()


# ---- queued entries (long segments): table entries a few steps beyond the ring reach whose
# slabs are read from the ring ahead of their use and held in registers (integer mode: two
# slots, distances in (384, 640] and (640, 1024]; interpolated mode: the first slot); in each
# segment's first steps they come from global memory. Rows checked: the first six steps of
# several segments, random rows, the end.

def ring_segment_len(BH, N, T=128):
    """Rows per segment of a ring-kernel launch (the library's ring_segments)."""
    tiles = -(-N // T)
    segs = -(-512 // BH)
    if -(-tiles // segs) < 8:
        segs = 256 // BH
    segs = max(1, min(segs, tiles))
    per = -(-tiles // segs)
    return per * T


QUEUED = [
    # (B, H, N, W, alpha, base)
    (1, 16, 40000, 12, 1.5, FIB_BASE),            # 566 and 915 queued, 1480 far
    (1, 8, 70000, 16, 1.0, (1, 2, 640, 1024)),     # both slots at their largest distances
    (1, 8, 70000, 16, 1.0, (1, 2, 385, 641)),      # at their smallest: a 256-row warm-up
    (2, 4, 50000, 12, 1.0, FIB_BASE + (1597, 2584)),  # two queued, two far
    (1, 8, 60000, 12, 1.0, tuple(range(20, 380, 25)) + (600, 900, 1300)),  # 15 covered
    (1, 8, 60000, 12, 1.0, (1, 2, 500, 1100, 1300)),  # slot 0 only, two far
    (1, 8, 60000, 12, 1.37, FIB_BASE),             # interpolated weights 0.51 (queued), ...
    (1, 8, 60000, 12, 1.0, (1, 2, 500)),           # one queued entry, no far entry
    (1, 8, 60000, 12, 1.0, (1, 2, 500, 1100)),     # one queued, one far
    (1, 8, 70000, 1, 1.5, FIB_BASE),               # W 1: 12 covered entries, then 566, 915, 1480
]


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("case", QUEUED, ids=[f"B{c[0]}H{c[1]}N{c[2]}W{c[3]}a{c[4]}n{len(c[5])}" for c in QUEUED])
def test_queued_entries(case, mode):
    B, H, N, W, alpha, base = case
    alpha = np.float32(alpha)
    seg = ring_segment_len(B * H, N)
    assert seg >= 8 * 128
    say("queued entries", case, "mode", mode, "segment rows", seg)
    qkv = inputs(5000 + N + W, (B, H, N, 64), BF16)
    o, lse = run_fwd(qkv, W, alpha, base, mode)
    n_seg = -(-N // seg)
    firsts = [seg * k for k in sorted({0, 1, 2, n_seg // 2, n_seg - 1})]
    rng = np.random.default_rng(N + W)
    rows = np.concatenate([np.arange(s, min(s + 6 * 128 + 8, N)) for s in firsts]
                          + [rng.integers(0, N, 200), np.arange(N - 40, N)])
    rows = np.unique(rows)
    (_, q64), (_, k64), (_, v64) = qkv[:3]
    eo = el = 0.0
    for b, h in [(0, 0), (B - 1, H - 1)]:
        ro, rl = O.forward_rows(q64[b, h], k64[b, h], v64[b, h], rows, W, alpha, base, 10000.0, mode)
        eo = max(eo, maxabs(host(o[b, h])[rows], ro))
        el = max(el, maxabs(host(lse[b, h])[rows], rl))
    say("  max err O", eo, "LSE", el, "rows", len(rows))
    assert eo <= TOL[BF16] and el <= TOL[BF16]
    assert torch.isfinite(o.float()).all().item()


@pytest.mark.parametrize("dtype", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_probe_moments(mode, dtype):
    """Q = 0 and V[j] = (j/N, (j/N)^2, 1, 0, ...): O_i[:3] is the mean of the attended
    positions, their second moment and 1 (closed form over an independently built attended
    set; interpolated keys at their fractional positions). bf16: the closed form uses the
    stored bf16 V values; the bound is the output's rounding (half an ulp below 1 is 2^-9)
    plus the rounding of the interpolation weights in the MFMA path."""
    from dense_reference import moment_probe_expected, moment_probe_v

    N, W, a = 1500, 12, np.float32(1.37)
    say("moment probe", mode, dtype)
    (_, _), (k, _), (_, _) = inputs(78, (1, 2, N, 64), dtype)
    vd = torch.from_numpy(np.broadcast_to(moment_probe_v(N), (1, 2, N, 64)).astype(np.float32).copy())
    vd = vd.cuda().to(k.dtype)
    o, _ = F.fwd(torch.zeros_like(k), k, vd, W, a, FIB_BASE, 10000.0, mode)
    oh = host(o)
    want = moment_probe_expected(N, W, a, FIB_BASE, mode == INTERP, vals=host(vd)[0, 0, :, :3])
    tol = 1e-5 if dtype == F32 else 2.0 ** -8
    for h in range(2):
        assert maxabs(oh[0, h, :, :3], want) <= tol
        assert np.abs(oh[0, h, :, 3:]).max() == 0.0


# the forward of small problems that the ring kernel does not take (fp32, or W > 16) runs on
# the gather kernel (every key of a query requested at once, 1-4 queries per block) up to 2^16
# query rows, on the general kernel above; both sides of the switch, both modes, 1, 2 and 4
# queries per block (the block size follows the window plus table size)
GATHER_SWITCH = [
    # (B, H, N, W, alpha, base, dtype)
    (1, 2, 32768, 12, 1.0, FIB_BASE, F32),     # 65536 rows: gather, 2 queries per block
    (1, 2, 32769, 12, 1.0, FIB_BASE, F32),     # 65538 rows: general kernel
    (2, 3, 700, 4, 0.77, (1, 2, 3, 5, 8, 13), F32),   # 4 queries per block
    (1, 1, 900, 40, 1.1, FIB_BASE, F32),       # 1 query per block, more keys than quads
    (2, 2, 600, 24, 0.93, POW2_BASE, BF16),    # bf16 with W > 16
]


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("case", GATHER_SWITCH,
                         ids=[f"B{c[0]}H{c[1]}N{c[2]}W{c[3]}a{c[4]}n{len(c[5])}d{c[6]}" for c in GATHER_SWITCH])
def test_gather_and_general_forward(case, mode):
    B, H, N, W, alpha, base, dtype = case
    say("gather / general forward", case, "mode", mode)
    qkv = inputs(6100 + N + W, (B, H, N, 64), dtype)
    check_full(qkv, W, np.float32(alpha), base, mode, dtype)
