"""Plain fp64 CPU oracle of causal Fibonacci-offset dilated sparse self-attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may use it. It shares no code, table or constant generator with the HIP library.

Source, cited below as [FIB]: "Depth-Staggered Fibonacci Spacing for Sparse Attention:
Static Schedules Beat Learned Dilation and Extrapolate Where Dense Attention Fails"
(arXiv 2606.28560), technical summaries on gist.science (Korean and Spanish pages, same
content). Sections used:
  * Method > Architecture and attention mechanism: attended set (dense local window of size
    W plus sparse offsets from fib = [1, 2, 3, 5, ..., 987]); scaling d_k = alpha * f_k with a
    per-layer alpha in [0.5, 1.5]; linear interpolation of key/value rows for non-integer
    offsets so that a gradient reaches alpha; RoPE applied before the gather.
  * Method > Experimental variables: the Fixed, Learned, Staggered-linear and
    Staggered-coprime (l -> 7l mod L) schedules over 16 layers.
  * Method > Controls: the reach-matched power-of-two base and the dense baseline.
  * Results 2 (learned dilation is inert), efficiency bullet: static (integer) offsets run on
    a fused boolean-mask path, non-integer ones on an interpolated gather.
  * Significance: vanilla RoPE without scaling.
The dropped-attention-mass diagnostic follows "SSA: Sparse Sparse Attention" (arXiv
2511.20102, gist.science Korean summary), 1. Problem definition, item 1 (attention gap): the
attention weight that full attention gives to keys the sparse mechanism does not select.

Readings taken where the pages leave a step open (each is the plainest one consistent with
the rest):
  R1 window = distances 0..W-1 (the query itself included); causal (keys j <= i).
  R2 the elided base list is the 15 distinct Fibonacci numbers 1..987.
  R3 integer mode rounds alpha*f half to even; the product is exact (alpha is the exact value
     of its fp32 bits). Offsets below W are dropped, equal offsets collapse (a set).
  R4 interpolated mode keeps entries with d >= W; c = ceil(d), lo = i - c, hi = lo + 1,
     weight w = c - d on hi and 1 - w on lo (w = 0 at integer d); an entry is valid for query
     i when c <= i. No deduplication.
  R5 RoPE: rotate-half pairs (j, j + D/2), omega_j = theta^(-2j/D), positions 0..N-1.
  R6 softmax scale 1/sqrt(D); O in the input dtype, LSE natural log.
  R7 V is interpolated with the same weight as K.
  R8 d(alpha) ignores the piecewise-constant dependence of c and of the kept set on alpha
     (both are locally constant), and is 0 in integer mode.
  R9 schedules: linear alpha_l = fp32 nearest to 0.5 + l/(L-1); coprime alpha_l =
     linear[(7 l) mod L]; fixed alpha = 1.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ProcessPoolExecutor
from fractions import Fraction

import numpy as np

INT = 0
INTERP = 1

__all__ = [
    "INT", "INTERP",
    "exact_alpha", "f32_nearest", "schedule_linear", "schedule_coprime",
    "int_offsets", "interp_entries", "rope_omega", "rope", "rope_inverse",
    "index_sets", "forward", "backward", "forward_rows",
    "dense_causal_lse", "dropped_mass", "DalphaScale",
]


# ---------------------------------------------------------------------------------------
# alpha: exact value of an fp32 number, and correct rounding of a rational to fp32
# ---------------------------------------------------------------------------------------

def exact_alpha(alpha) -> Fraction:
    """Exact rational value of alpha rounded to fp32 (the per-layer scalar of [FIB] Method)."""
    a = np.float32(alpha)
    if not np.isfinite(a):
        raise ValueError("alpha must be finite")
    return Fraction(float(a))


def f32_nearest(x: Fraction) -> np.float32:
    """The fp32 value nearest to the rational x, ties to an even significand."""
    x = Fraction(x)
    guess = np.float32(float(x))
    cands = {guess, np.nextafter(guess, np.float32(np.inf)), np.nextafter(guess, np.float32(-np.inf))}
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        dist = abs(Fraction(float(c)) - x)
        even = (int(np.asarray(c, dtype=np.float32).view(np.uint32)) & 1) == 0
        key = (dist, 0 if even else 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def schedule_linear(n_layers: int = 16):
    """Staggered-linear schedule ([FIB] Experimental variables, item 3): alpha ramps linearly
    from 0.5 at layer 0 to 1.5 at the last layer; each value is the nearest fp32."""
    if n_layers < 2:
        raise ValueError("a linear ramp needs at least 2 layers")
    L1 = n_layers - 1
    return [f32_nearest(Fraction(1, 2) + Fraction(l, L1)) for l in range(n_layers)]


def schedule_coprime(n_layers: int = 16, stride: int = 7):
    """Staggered-coprime schedule ([FIB] Experimental variables, item 4): the linear ramp's
    alpha multiset reassigned with the coprime stride l -> stride*l mod L. Reading: layer l
    takes the ramp value at index stride*l mod L (for L = 16 the map is its own inverse)."""
    if math.gcd(stride, n_layers) != 1:
        raise ValueError("stride must be coprime to the layer count")
    lin = schedule_linear(n_layers)
    return [lin[(stride * l) % n_layers] for l in range(n_layers)]


# ---------------------------------------------------------------------------------------
# offset table ([FIB] Method > Architecture: d_k = alpha * f_k; Results 2: integer offsets
# for static schedules, interpolation for non-integer ones)
# ---------------------------------------------------------------------------------------

def _round_half_even(x: Fraction) -> int:
    fl = math.floor(x)
    rem = x - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def _check_base(base):
    base = [int(f) for f in base]
    if not base:
        raise ValueError("empty base")
    if any(f <= 0 for f in base):
        raise ValueError("base entries must be positive")
    if any(b <= a for a, b in zip(base, base[1:])):
        raise ValueError("base must be strictly increasing")
    return base


def int_offsets(alpha, base, W: int):
    """Integer mode: r_k = round_half_even(alpha * f_k); keep r_k >= W; as a sorted set."""
    a = exact_alpha(alpha)
    base = _check_base(base)
    kept = set()
    for f in base:
        r = _round_half_even(a * f)
        if r >= W:
            kept.add(r)
    return sorted(kept)


def interp_entries(alpha, base, W: int):
    """Interpolated mode: for each f_k with d_k = alpha*f_k >= W, the entry
    (f_k, c_k = ceil(d_k), w_k = c_k - d_k) with w_k an exact Fraction in [0, 1)."""
    a = exact_alpha(alpha)
    base = _check_base(base)
    out = []
    for f in base:
        d = a * f
        if d >= W:
            c = math.ceil(d)
            out.append((f, c, c - d))
    return out


# ---------------------------------------------------------------------------------------
# RoPE ([FIB] Method > Architecture: applied before the gather; Significance: vanilla RoPE)
# ---------------------------------------------------------------------------------------

def rope_omega(D: int, theta: float) -> np.ndarray:
    """omega_j = theta^(-2j/D), j < D/2, in fp64."""
    j = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / D)


def rope(x: np.ndarray, theta: float, positions=None) -> np.ndarray:
    """Rotate-half RoPE of rows x[..., p, :] at positions p (default 0..N-1), fp64."""
    x = np.asarray(x, dtype=np.float64)
    N, D = x.shape[-2], x.shape[-1]
    pos = np.arange(N, dtype=np.float64) if positions is None else np.asarray(positions, dtype=np.float64)
    phi = pos[:, None] * rope_omega(D, theta)[None, :]
    c, s = np.cos(phi), np.sin(phi)
    h = D // 2
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rope_inverse(x: np.ndarray, theta: float, positions=None) -> np.ndarray:
    """Transpose (inverse) of ``rope``: rotation by -p*omega_j."""
    x = np.asarray(x, dtype=np.float64)
    N, D = x.shape[-2], x.shape[-1]
    pos = np.arange(N, dtype=np.float64) if positions is None else np.asarray(positions, dtype=np.float64)
    phi = pos[:, None] * rope_omega(D, theta)[None, :]
    c, s = np.cos(phi), np.sin(phi)
    h = D // 2
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c + hi * s, hi * c - lo * s], axis=-1)


# ---------------------------------------------------------------------------------------
# attended rows of every query
# ---------------------------------------------------------------------------------------

def index_sets(N: int, W: int, alpha, base, mode: int) -> np.ndarray:
    """Per-query attended rows as an int32 [N, W + n_entries] array, -1 where absent.

    Column s < W: window key i - s. Column W + e: table entry e (sorted offsets in integer
    mode, kept base entries in base order in interpolated mode): row i - r_e, or the lower
    row i - c_e of the interpolated pair.
    """
    if mode == INT:
        dist = int_offsets(alpha, base, W)
    else:
        dist = [c for _, c, _ in interp_entries(alpha, base, W)]
    out = np.full((N, W + len(dist)), -1, dtype=np.int32)
    for i in range(N):
        for s in range(min(W, i + 1)):
            out[i, s] = i - s
        for e, d in enumerate(dist):
            if d <= i:
                out[i, W + e] = i - d
    return out


# ---------------------------------------------------------------------------------------
# forward / backward of one (b, h) head, vectorised over query chunks
# ---------------------------------------------------------------------------------------

def _head_plan(N: int, W: int, alpha, base, mode: int):
    """Gather plan: for every query, the virtual keys as (lo, hi, w, f) arrays [N, S]."""
    if mode == INT:
        offs = int_offsets(alpha, base, W)
        dist = np.array(offs, dtype=np.int64)
        wts = np.zeros(len(offs))
        fs = np.zeros(len(offs))
        hi_shift = np.zeros(len(offs), dtype=np.int64)
    elif mode == INTERP:
        ent = interp_entries(alpha, base, W)
        dist = np.array([c for _, c, _ in ent], dtype=np.int64)
        wts = np.array([float(w) for _, _, w in ent], dtype=np.float64)
        fs = np.array([f for f, _, _ in ent], dtype=np.float64)
        hi_shift = np.ones(len(ent), dtype=np.int64)
    else:
        raise ValueError("mode must be INT or INTERP")
    return dist, wts, fs, hi_shift


def _gather(rows_i, W, dist, wts, hi_shift):
    """lo/hi/weight/valid arrays [n, W + n_entries] for the query rows rows_i."""
    i = rows_i[:, None]
    win_lo = i - np.arange(W, dtype=np.int64)[None, :]
    win_valid = win_lo >= 0
    off_lo = i - dist[None, :]
    off_valid = off_lo >= 0
    lo = np.concatenate([win_lo, off_lo], axis=1)
    hi = np.concatenate([win_lo, off_lo + hi_shift[None, :]], axis=1)
    w = np.concatenate([np.zeros((1, W)), wts[None, :]], axis=1) * np.ones_like(lo, dtype=np.float64)
    valid = np.concatenate([win_valid, off_valid], axis=1)
    lo = np.where(valid, lo, 0)
    hi = np.where(valid, hi, 0)
    return lo, hi, w, valid


def _chunk(n_keys: int, D: int) -> int:
    return max(1, min(4096, (48 << 20) // max(1, 8 * n_keys * D * 4)))


def _head_forward(qh, kh, vh, W, alpha, base, theta, mode, rows=None):
    N, D = qh.shape
    qr = rope(qh, theta)
    kr = rope(kh, theta)
    vh = np.asarray(vh, dtype=np.float64)
    dist, wts, _, hi_shift = _head_plan(N, W, alpha, base, mode)
    scale = 1.0 / math.sqrt(D)
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((len(rows), D))
    LSE = np.zeros(len(rows))
    step = _chunk(W + len(dist), D)
    for a in range(0, len(rows), step):
        ri = rows[a:a + step]
        lo, hi, w, valid = _gather(ri, W, dist, wts, hi_shift)
        key = (1.0 - w)[..., None] * kr[lo] + w[..., None] * kr[hi]
        val = (1.0 - w)[..., None] * vh[lo] + w[..., None] * vh[hi]
        s = np.einsum("nd,nsd->ns", qr[ri], key) * scale
        s = np.where(valid, s, -np.inf)
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        O[a:a + step] = np.einsum("ns,nsd->nd", p, val) / l[:, None]
        LSE[a:a + step] = m + np.log(l)
    return O, LSE


def _head_backward(qh, kh, vh, doh, W, alpha, base, theta, mode, rows=None):
    """Hand-derived backward of one head; returns dq, dk, dv, dalpha (fp64).

    With s = <q^, key>/sqrt(D), P = softmax(s) over the attended set, O = sum P*value:
      Delta_i = <dO_i, O_i>, dP_ik = <dO_i, value_k>, dS_ik = P_ik (dP_ik - Delta_i),
      dq^_i = sum_k dS_ik key_k / sqrt(D), dkey_k += dS_ik q^_i / sqrt(D), dvalue_k += P_ik dO_i,
    interpolated keys split dkey/dvalue onto lo with 1 - w and onto hi with w, and since
    w = c - alpha*f, d w / d alpha = -f gives
      dalpha = sum_ik -f_k [dS_ik <q^_i, k^_hi - k^_lo>/sqrt(D) + P_ik <dO_i, v_hi - v_lo>].
    Rotations are undone at the end: dQ_i = R_i^T dq^_i, dK_j = R_j^T dk^_j.
    ``rows`` restricts the queries whose contributions are summed (default: all).

    Besides dalpha, four sums over queries i describe its size and conditioning (they enter
    no result): with t_i = sum_k -f_k g_ik the query's contribution,
      sum |t_i|, sum t_i^2, sum a_i^2 with a_i = sum_k f_k (|dS_ik ds_ik| + P_ik |ddp_ik|)
      (ds = s_hi - s_lo, ddp = dp_hi - dp_lo), and sum b_i^2 with
      b_i = sum_k f_k P_ik ((|dP_ik| + |Delta_i|)(|s_hi| + |s_lo|) + |dp_hi| + |dp_lo|),
    the magnitudes of the parts whose rounding errors make up the error of t_i.
    """
    N, D = qh.shape
    qr = rope(qh, theta)
    kr = rope(kh, theta)
    vh = np.asarray(vh, dtype=np.float64)
    doh = np.asarray(doh, dtype=np.float64)
    dist, wts, fs, hi_shift = _head_plan(N, W, alpha, base, mode)
    scale = 1.0 / math.sqrt(D)
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    dqr = np.zeros((N, D))
    dkr = np.zeros((N, D))
    dv = np.zeros((N, D))
    dalpha = 0.0
    sums = np.zeros(4)  # sum |t_i|, sum t_i^2, sum a_i^2, sum b_i^2 (see above)
    S = W + len(dist)
    fk = np.concatenate([np.zeros(W), fs])
    step = _chunk(S, D)
    for a in range(0, len(rows), step):
        ri = rows[a:a + step]
        lo, hi, w, valid = _gather(ri, W, dist, wts, hi_shift)
        key = (1.0 - w)[..., None] * kr[lo] + w[..., None] * kr[hi]
        val = (1.0 - w)[..., None] * vh[lo] + w[..., None] * vh[hi]
        q = qr[ri]
        do = doh[ri]
        s = np.einsum("nd,nsd->ns", q, key) * scale
        s = np.where(valid, s, -np.inf)
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        p = p / p.sum(axis=1)[:, None]
        o = np.einsum("ns,nsd->nd", p, val)
        delta = np.einsum("nd,nd->n", do, o)
        dp = np.einsum("nd,nsd->ns", do, val)
        ds = np.where(valid, p * (dp - delta[:, None]), 0.0)
        dqr[ri] += np.einsum("ns,nsd->nd", ds, key) * scale
        dkey = ds[..., None] * q[:, None, :] * scale
        dval = p[..., None] * do[:, None, :]
        # scatter per key slot: within one slot the rows lo (and hi) of distinct queries are
        # distinct, so a plain indexed add is exact
        for col in range(S):
            mcol = valid[:, col]
            if not mcol.any():
                continue
            lo_c, hi_c, w_c = lo[mcol, col], hi[mcol, col], w[mcol, col][:, None]
            for tgt, src in ((dkr, dkey), (dv, dval)):
                tgt[lo_c] += (1.0 - w_c) * src[mcol, col]
                tgt[hi_c] += w_c * src[mcol, col]
        if mode == INTERP:
            dk_diff = np.einsum("nd,nsd->ns", q, kr[hi] - kr[lo]) * scale
            dv_diff = np.einsum("nd,nsd->ns", do, vh[hi] - vh[lo])
            g = ds * dk_diff + p * dv_diff
            per_query = np.sum(np.where(valid, -fk[None, :] * g, 0.0), axis=1)
            dalpha += float(np.sum(per_query))
            a_i = np.sum(np.where(valid, fk[None, :] * (np.abs(ds * dk_diff) + p * np.abs(dv_diff)), 0.0), axis=1)
            s_lo = np.einsum("nd,nsd->ns", q, kr[lo]) * scale
            s_hi = np.einsum("nd,nsd->ns", q, kr[hi]) * scale
            dp_lo = np.einsum("nd,nsd->ns", do, vh[lo])
            dp_hi = np.einsum("nd,nsd->ns", do, vh[hi])
            b_terms = p * ((np.abs(dp) + np.abs(delta)[:, None]) * (np.abs(s_hi) + np.abs(s_lo))
                           + np.abs(dp_hi) + np.abs(dp_lo))
            b_i = np.sum(np.where(valid, fk[None, :] * b_terms, 0.0), axis=1)
            sums += [np.sum(np.abs(per_query)), np.sum(per_query ** 2), np.sum(a_i ** 2), np.sum(b_i ** 2)]
    dq = rope_inverse(dqr, theta)
    dk = rope_inverse(dkr, theta)
    return dq, dk, dv, dalpha, sums


def _bh_iter(x):
    B, H = x.shape[0], x.shape[1]
    for b in range(B):
        for h in range(H):
            yield b, h


def _fwd_task(args):
    return _head_forward(*args)


def _bwd_task(args):
    return _head_backward(*args)


def _workers(workers):
    if workers is None:
        return 1
    if workers == 0:
        return len(os.sched_getaffinity(0))
    return int(workers)


def forward(q, k, v, W, alpha, base, theta=10000.0, mode=INT, workers=1):
    """O [B,H,N,D] and LSE [B,H,N] (fp64) of the sparse attention; inputs [B,H,N,D].

    ``workers`` > 1 (0 = all cores in the affinity mask) runs the independent (b, h) heads
    in a process pool.
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    if W < 1:
        raise ValueError("W must be >= 1")
    B, H, N, D = q.shape
    O = np.zeros_like(q)
    LSE = np.zeros((B, H, N))
    jobs = [(q[b, h], k[b, h], v[b, h], W, alpha, base, theta, mode) for b, h in _bh_iter(q)]
    nw = _workers(workers)
    if nw > 1 and len(jobs) > 1:
        with ProcessPoolExecutor(max_workers=min(nw, len(jobs))) as ex:
            res = list(ex.map(_fwd_task, jobs))
    else:
        res = [_fwd_task(j) for j in jobs]
    for (b, h), (o, lse) in zip(_bh_iter(q), res):
        O[b, h] = o
        LSE[b, h] = lse
    return O, LSE


def forward_rows(qh, kh, vh, rows, W, alpha, base, theta=10000.0, mode=INT):
    """O and LSE of selected query rows of one head (inputs [N, D]); for sampled checks."""
    return _head_forward(qh, kh, vh, W, alpha, base, theta, mode, rows=rows)


class DalphaScale(tuple):
    """Size of dalpha's summands over all queries (see _head_backward): sum_abs = sum |t_i|,
    rss_query = sqrt(sum t_i^2), rss_entry = sqrt(sum a_i^2), rss_wide = sqrt(sum b_i^2)."""

    __slots__ = ()

    def __new__(cls, sums):
        return tuple.__new__(cls, (float(sums[0]), math.sqrt(sums[1]), math.sqrt(sums[2]), math.sqrt(sums[3])))

    sum_abs = property(lambda self: self[0])
    rss_query = property(lambda self: self[1])
    rss_entry = property(lambda self: self[2])
    rss_wide = property(lambda self: self[3])


def backward(q, k, v, dout, W, alpha, base, theta=10000.0, mode=INT, workers=1, rows=None, return_scale=False):
    """dQ, dK, dV [B,H,N,D] (fp64, w.r.t. the un-rotated inputs) and dalpha (float).

    With ``return_scale`` a fifth value is returned, a DalphaScale: the sizes of the per-query
    contributions to dalpha and of their parts (all zero in integer mode), against which an
    approximate dalpha's error can be judged when the contributions cancel.
    """
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    B, H, N, D = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(q)
    dv = np.zeros_like(q)
    dalpha = 0.0
    sums = np.zeros(4)
    jobs = [(q[b, h], k[b, h], v[b, h], dout[b, h], W, alpha, base, theta, mode, rows)
            for b, h in _bh_iter(q)]
    nw = _workers(workers)
    if nw > 1 and len(jobs) > 1:
        with ProcessPoolExecutor(max_workers=min(nw, len(jobs))) as ex:
            res = list(ex.map(_bwd_task, jobs))
    else:
        res = [_bwd_task(j) for j in jobs]
    for (b, h), (a, bb, c, da, hs) in zip(_bh_iter(q), res):
        dq[b, h] = a
        dk[b, h] = bb
        dv[b, h] = c
        dalpha += da
        sums += hs
    if return_scale:
        return dq, dk, dv, dalpha, DalphaScale(sums)
    return dq, dk, dv, dalpha


# ---------------------------------------------------------------------------------------
# dense causal attention and the mass it puts outside the sparse set (diagnostic)
# ---------------------------------------------------------------------------------------

def dense_causal_lse(q, k, theta=10000.0):
    """LSE [..., N] (natural log, fp64) of dense causal attention logits: for query i, log of
    the sum over keys j <= i of exp(<R_i q_i, R_j k_j> / sqrt(D)); inputs [..., N, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N, D = q.shape[-2], q.shape[-1]
    qr, kr = rope(q, theta), rope(k, theta)
    s = np.matmul(qr, np.swapaxes(kr, -1, -2)) / math.sqrt(D)
    future = np.triu(np.ones((N, N), dtype=bool), k=1)
    s = np.where(future, -np.inf, s)
    m = np.max(s, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(s - m), axis=-1, keepdims=True)))[..., 0]


def dropped_mass(q, k, W, alpha, base, theta=10000.0):
    """Per query, the dense causal softmax mass on keys outside the integer-mode attended set
    (window plus kept offsets): 1 - sum over j in S_i of softmax_dense(i, j). Inputs
    [..., N, D]; output [..., N] in fp64. (Interpolated entries blend two rows, so the set is
    defined for integer offsets only.)"""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N, D = q.shape[-2], q.shape[-1]
    qr, kr = rope(q, theta), rope(k, theta)
    s = np.matmul(qr, np.swapaxes(kr, -1, -2)) / math.sqrt(D)
    future = np.triu(np.ones((N, N), dtype=bool), k=1)
    s = np.where(future, -np.inf, s)
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    p = p / np.sum(p, axis=-1, keepdims=True)
    inset = np.zeros((N, N), dtype=bool)
    rows = index_sets(N, W, alpha, base, INT)
    for i in range(N):
        cols = rows[i][rows[i] >= 0]
        inset[i, cols] = True
    return 1.0 - np.sum(np.where(inset, p, 0.0), axis=-1)
