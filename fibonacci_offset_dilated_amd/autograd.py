"""torch.autograd wrapper of the sparse attention op and the Learned-schedule parameter.

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

``LearnedDilation`` is the per-layer free parameter theta of the Learned schedule. The pages
give no map from theta to alpha beyond alpha in [0.5, 1.5] initialised at 1; this module
uses alpha = 1 + 0.5 tanh(theta) (theta = 0 gives alpha = 1; the range is the open interval
(0.5, 1.5)).
"""
from __future__ import annotations

from typing import Sequence

import numpy as np
import torch

from ._lib import INTERP, bwd, bwd_dev, fwd, fwd_dev

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
