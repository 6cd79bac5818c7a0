"""Independent dense formulations used to pin the oracle on tiny inputs.

Nothing here imports the oracle or the HIP library. The attended set is rebuilt from a
brute-force membership predicate over integer distances, RoPE is written as a complex
multiplication, and attention runs through torch (fp64, CPU): scaled_dot_product_attention
with an explicit boolean mask for integer mode, and a dense "augmented key" formulation
(interpolated logits as linear combinations of dense logits) for interpolated mode. Both are
differentiable, so torch autograd gives reference gradients, d(alpha) included.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch


def exact(alpha) -> Fraction:
    return Fraction(float(np.float32(alpha)))


def int_member(delta: int, alpha, base, W: int) -> bool:
    """Is integer distance delta an attended offset in integer mode?

    delta is attended when delta >= W and some alpha*f lies strictly within 1/2 of delta, or
    exactly 1/2 away with delta even (ties go to the even integer).
    """
    if delta < W:
        return False
    a = exact(alpha)
    for f in base:
        gap = abs(a * f - delta)
        if gap < Fraction(1, 2) or (gap == Fraction(1, 2) and delta % 2 == 0):
            return True
    return False


def int_mask(N: int, W: int, alpha, base) -> np.ndarray:
    """Boolean [N, N] mask M[i, j]: 0 <= j <= i and (i - j < W or i - j is an offset)."""
    max_d = N
    offs = {d for d in range(max_d) if int_member(d, alpha, base, W)}
    M = np.zeros((N, N), dtype=bool)
    for i in range(N):
        for j in range(i + 1):
            d = i - j
            M[i, j] = d < W or d in offs
    return M


def interp_virtuals(alpha, base, W: int):
    """(f, lo_distance, hi_distance, w) for every base entry with alpha*f >= W.

    lo_distance is the smallest integer c with c >= alpha*f; the virtual key sits at
    distance alpha*f = c - w between rows at distances c (weight 1 - w) and c - 1 (weight w).
    """
    a = exact(alpha)
    out = []
    for f in base:
        d = a * f
        if d < W:
            continue
        c = int(d)
        if c < d:
            c += 1
        out.append((f, c, c - 1, float(c - d)))
    return out


def rope_complex(x: torch.Tensor, theta: float) -> torch.Tensor:
    """RoPE as complex multiplication: z_j = x_j + i x_{j+D/2}, z_j * exp(i p theta^(-2j/D))."""
    N, D = x.shape[-2], x.shape[-1]
    h = D // 2
    z = torch.complex(x[..., :h], x[..., h:])
    j = torch.arange(h, dtype=torch.float64)
    freq = torch.tensor(float(theta), dtype=torch.float64) ** (-2.0 * j / D)
    p = torch.arange(N, dtype=torch.float64)
    rot = torch.polar(torch.ones(N, h, dtype=torch.float64), p[:, None] * freq[None, :])
    zr = z * rot
    return torch.cat([zr.real, zr.imag], dim=-1)


def dense_int_forward(q, k, v, W, alpha, base, theta=10000.0):
    """Integer mode via torch SDPA under the brute-force mask; returns O, LSE (fp64)."""
    q, k, v = (torch.as_tensor(t, dtype=torch.float64) for t in (q, k, v))
    N, D = q.shape[-2], q.shape[-1]
    M = torch.as_tensor(int_mask(N, W, alpha, base))
    qr, kr = rope_complex(q, theta), rope_complex(k, theta)
    O = torch.nn.functional.scaled_dot_product_attention(qr, kr, v, attn_mask=M)
    s = (qr @ kr.transpose(-1, -2)) / math.sqrt(D)
    s = s.masked_fill(~M, float("-inf"))
    LSE = torch.logsumexp(s, dim=-1)
    return O, LSE


def dense_augmented(q, k, v, W, alpha_t, base, theta=10000.0):
    """Interpolated mode as a dense formulation differentiable in q, k, v and alpha_t.

    Dense logits S = rot(Q) rot(K)^T / sqrt(D). For query i the window logits are S[i, j],
    i - W < j <= i; each virtual key (c, w) valid for i (c <= i) has logit
    (1 - w) S[i, i - c] + w S[i, i - c + 1] and value (1 - w) V[i - c] + w V[i - c + 1],
    with w = c - alpha * f so that alpha carries a gradient.
    Returns O [.., N, D] and LSE [.., N].
    """
    q, k, v = (torch.as_tensor(t, dtype=torch.float64) for t in (q, k, v))
    N, D = q.shape[-2], q.shape[-1]
    qr, kr = rope_complex(q, theta), rope_complex(k, theta)
    S = (qr @ kr.transpose(-1, -2)) / math.sqrt(D)
    virt = interp_virtuals(float(alpha_t.detach()), base, W)
    outs, lses = [], []
    for i in range(N):
        logits, values = [], []
        for j in range(max(0, i - W + 1), i + 1):
            logits.append(S[..., i, j])
            values.append(v[..., j, :])
        for f, c, _, _ in virt:
            if c > i:
                continue
            w = c - alpha_t * f
            lo, hi = i - c, i - c + 1
            logits.append((1 - w) * S[..., i, lo] + w * S[..., i, hi])
            values.append((1 - w) * v[..., lo, :] + w * v[..., hi, :])
        lg = torch.stack(logits, dim=-1)
        vals = torch.stack(values, dim=-2)
        p = torch.softmax(lg, dim=-1)
        outs.append((p[..., None] * vals).sum(dim=-2))
        lses.append(torch.logsumexp(lg, dim=-1))
    return torch.stack(outs, dim=-2), torch.stack(lses, dim=-1)


def moment_probe_v(N: int, D: int = 64, vrow=None) -> np.ndarray:
    """V rows (x_j, x_j^2, 1, 0, ...) with x_j = vrow[j] (default j / N), [N, D] fp64."""
    x = np.arange(N, dtype=np.float64) / N if vrow is None else np.asarray(vrow, dtype=np.float64)
    v = np.zeros((N, D))
    v[:, 0], v[:, 1], v[:, 2] = x, x ** 2, 1.0
    return v


def moment_probe_expected(N: int, W: int, alpha, base, interp: bool, vals=None) -> np.ndarray:
    """Closed form of the moment probe, [N, 3]: with Q = 0 every attended (virtual) key of
    query i gets the same weight, so O_i[:3] is the plain average over its attended set of
    the first three V columns: vals [N, 3] (default (j/N, (j/N)^2, 1), moment_probe_v's rows).
    Integer mode: the window and the distances that int_member accepts (<= i). Interpolated
    mode: the window plus, for each entry of interp_virtuals with c <= i,
    (1 - w) V[i - c] + w V[i - c + 1]."""
    vals = moment_probe_v(N)[:, :3] if vals is None else np.asarray(vals, dtype=np.float64)
    row = lambda j: vals[j]
    offs = [] if interp else [d for d in range(W, N) if int_member(d, alpha, base, W)]
    virt = interp_virtuals(alpha, base, W) if interp else []
    out = np.zeros((N, 3))
    for i in range(N):
        terms = [row(i - s) for s in range(min(W, i + 1))]
        terms += [row(i - d) for d in offs if d <= i]
        terms += [(1 - w) * row(i - c) + w * row(i - c + 1) for _, c, _, w in virt if c <= i]
        out[i] = np.mean(terms, axis=0)
    return out
