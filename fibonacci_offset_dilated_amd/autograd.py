"""torch.autograd wrapper of the sparse attention op, the Learned-schedule parameter and an
attention layer with its projections.

The attention layer of "Depth-Staggered Fibonacci Spacing for Sparse Attention" (gist.science
summaries of arXiv 2606.28560, Method > Architecture and attention mechanism; Method >
Experimental variables for the Learned schedule): ``fib_sparse_attention`` runs the forward
kernel and, in the backward pass, the backward kernel, which returns dL/dq, dL/dk, dL/dv and
dL/dalpha (the interpolated offsets are what let the gradient reach alpha; in integer mode
the offsets are piecewise constant in alpha and dL/dalpha is 0).

alpha is either a host float, or a one-element tensor. A float32 tensor on the inputs'
device together with an ``alpha_range`` = (lo, hi) stays on the device: the device-alpha
entry points build the offset table on the GPU, so the call involves no host copy of alpha
and no stream synchronization. Any other tensor is read once per call on the host.

``FibSparseSelfAttention`` is the attention sub-layer of the pages' models (Method >
Architecture and attention mechanism: hidden 512 = 8 heads x 64): a bias-free QKV projection,
the sparse attention (RoPE inside the op) and a bias-free output projection; the projections
are plain library GEMMs (torch.nn.Linear).

``LearnedDilation`` is the per-layer free parameter theta of the Learned schedule. The pages
give no map from theta to alpha beyond alpha in [0.5, 1.5] initialised at 1; this module
uses alpha = 1 + 0.5 tanh(theta) (theta = 0 gives alpha = 1; the range is the open interval
(0.5, 1.5)).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from ._lib import INT, INTERP, bwd, bwd_dev, fwd, fwd_dev

FIB_BASE_987 = (1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987)


def _alpha_value(alpha) -> np.float32:
    if isinstance(alpha, torch.Tensor):
        if alpha.numel() != 1:
            raise ValueError("alpha must hold one value")
        return np.float32(alpha.detach().to(torch.float32).cpu().item())
    return np.float32(alpha)


def _on_device(alpha, q, alpha_range) -> bool:
    return (alpha_range is not None and isinstance(alpha, torch.Tensor) and alpha.dtype == torch.float32
            and alpha.numel() == 1 and alpha.device == q.device)


class FibSparseAttentionFn(torch.autograd.Function):
    """O = attention(q, k, v; W, alpha, base, theta, mode); gradients for q, k, v and alpha."""

    @staticmethod
    def forward(ctx, q, k, v, alpha, W: int, base: Sequence[int], theta: float, mode: int, alpha_range):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        dev = _on_device(alpha, q, alpha_range)
        if dev:
            a = alpha.detach().reshape(1).contiguous()
            o, lse = fwd_dev(q, k, v, W, a, alpha_range, base, theta, mode)
            ctx.save_for_backward(q, k, v, o, lse, a)
        else:
            a = _alpha_value(alpha)
            o, lse = fwd(q, k, v, W, a, base, theta, mode)
            ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (W, None if dev else a, tuple(base), float(theta), int(mode), alpha_range if dev else None)
        ctx.alpha_is_tensor = isinstance(alpha, torch.Tensor)
        ctx.alpha_meta = (alpha.shape, alpha.dtype, alpha.device) if ctx.alpha_is_tensor else None
        return o

    @staticmethod
    def backward(ctx, do):
        W, a, base, theta, mode, alpha_range = ctx.cfg
        want_alpha = ctx.alpha_is_tensor and ctx.needs_input_grad[3]
        if alpha_range is not None:
            q, k, v, o, lse, adev = ctx.saved_tensors
            dq, dk, dv, da = bwd_dev(q, k, v, o, lse, do.contiguous(), W, adev, alpha_range, base, theta, mode,
                                     want_dalpha=want_alpha)
        else:
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv, da = bwd(q, k, v, o, lse, do.contiguous(), W, a, base, theta, mode, want_dalpha=want_alpha)
        dalpha = None
        if want_alpha:
            shape, dtype, device = ctx.alpha_meta
            dalpha = da.reshape(shape).to(device=device, dtype=dtype)
        return dq, dk, dv, dalpha, None, None, None, None, None


def fib_sparse_attention(q, k, v, alpha, W: int = 12, base: Sequence[int] = FIB_BASE_987, theta: float = 10000.0,
                         mode: int = INTERP, alpha_range=None):
    """Sparse attention over [B, H, N, 64] q, k, v (un-rotated; RoPE is applied inside).

    alpha: a float or a one-element tensor; when it is a tensor that requires grad, the
    backward pass fills its gradient (interpolated mode). With alpha a float32 tensor on the
    inputs' device and alpha_range = (lo, hi) bounding it, alpha never leaves the device."""
    rng = None if alpha_range is None else (float(alpha_range[0]), float(alpha_range[1]))
    return FibSparseAttentionFn.apply(q, k, v, alpha, int(W), tuple(base), float(theta), int(mode), rng)


class LearnedDilation(torch.nn.Module):
    """Per-layer dilation alpha = 1 + 0.5 tanh(theta) with theta a free parameter (init 0,
    i.e. alpha = 1), for the Learned schedule."""

    def __init__(self):
        super().__init__()
        self.theta = torch.nn.Parameter(torch.zeros(1))

    def alpha(self) -> torch.Tensor:
        return 1.0 + 0.5 * torch.tanh(self.theta)

    def forward(self, q, k, v, W: int = 12, base: Sequence[int] = FIB_BASE_987, rope_theta: float = 10000.0):
        # alpha lies in [0.5, 1.5] by construction, so it can stay on the device
        return fib_sparse_attention(q, k, v, self.alpha(), W, base, rope_theta, INTERP, alpha_range=(0.5, 1.5))


class FibSparseSelfAttention(torch.nn.Module):
    """x [B, N, hidden] -> Linear(hidden, 3 hidden) -> per-head q, k, v [B, H, N, D] -> sparse
    attention -> Linear(hidden, hidden). ``alpha``: a fixed per-layer float (static schedules:
    integer offsets by default), or "learned" (a LearnedDilation parameter, interpolated
    offsets, alpha kept on the device)."""

    def __init__(self, hidden: int = 512, heads: int = 8, W: int = 12, alpha=1.0,
                 base: Sequence[int] = FIB_BASE_987, rope_theta: float = 10000.0, mode: Optional[int] = None):
        super().__init__()
        if hidden % heads != 0 or hidden // heads != 64:
            raise ValueError("head size hidden / heads must be 64")
        self.heads, self.W, self.base, self.rope_theta = heads, int(W), tuple(base), float(rope_theta)
        self.qkv = torch.nn.Linear(hidden, 3 * hidden, bias=False)
        self.out = torch.nn.Linear(hidden, hidden, bias=False)
        self.learned = isinstance(alpha, str) and alpha == "learned"
        if self.learned:
            self.dilation = LearnedDilation()
            self.mode = INTERP if mode is None else int(mode)
        else:
            self.alpha = float(alpha)
            self.mode = INT if mode is None else int(mode)

    def forward(self, x):
        B, N, C = x.shape
        H = self.heads
        qkv = self.qkv(x).view(B, N, 3, H, C // H).permute(2, 0, 3, 1, 4)
        q, k, v = (t.contiguous() for t in qkv)
        if self.learned:
            a = self.dilation.alpha()
            o = fib_sparse_attention(q, k, v, a, self.W, self.base, self.rope_theta, self.mode, alpha_range=(0.5, 1.5))
        else:
            o = fib_sparse_attention(q, k, v, self.alpha, self.W, self.base, self.rope_theta, self.mode)
        return self.out(o.transpose(1, 2).reshape(B, N, C))
