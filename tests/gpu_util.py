"""Shared helpers of the GPU parity tests: seeded inputs on both sides, tolerances."""
from __future__ import annotations

import sys

import numpy as np

from fibonacci_offset_dilated_amd.synthetic import bf16_bits_to_f32, f32_to_bf16_bits, normal_inputs
from fibonacci_offset_dilated_amd.workloads import BF16, F32

# max-abs error bounds on O and LSE (fp32 accumulation in the kernels)
TOL = {F32: 1e-4, BF16: 2e-2}
# gradients are stored in the input dtype and reach magnitudes where one rounding step of
# the output alone exceeds the flat bound (bf16 half-ulp at |x| in [8, 16) is 2^-5), so the
# bound on dQ, dK, dV is the flat bound plus one ulp of the reference value:
#   |got - ref| <= TOL + REL_ULP * |ref|   (REL_ULP = 2^-7 for bf16, 2^-23 for fp32)
REL_ULP = {F32: 2.0 ** -23, BF16: 2.0 ** -7}
# bound on dalpha. dalpha = sum_i t_i over queries, and t_i = sum over the query's table
# entries of parts f dS (s_hi - s_lo) and f P (dp_hi - dp_lo). The computed parts carry a few
# rounding errors of the arithmetic's unit relative to their own size (bf16 operands: 2^-8;
# fp32 arithmetic: 2^-24 per operation, a few dozen per 64-term dot product, 2^-20), so the
# error of t_i is a few units times a_i = sum_k |parts| (oracle DalphaScale, rss_entry =
# sqrt(sum a_i^2)). Roundings to nearest even are unbiased and those of different queries
# independent, so the error of the sum grows like sqrt(sum a_i^2), not like sum a_i:
#   |got - ref| <= C[dtype] * rss_entry + 2^-18 * sum_i |t_i|
# The second term bounds the fp32 accumulation of the per-query terms (at most 64 terms per
# running sum before a fixed-order tree in the kernels: 64 * 2^-24 = 2^-18 relative to the
# sum of the magnitudes).
DALPHA_C = {F32: 2.5 * 2.0 ** -20, BF16: 2.5 * 2.0 ** -8}
DALPHA_ACC = 2.0 ** -18


def dalpha_bound(scale, dtype: int, factor: float = 1.0) -> float:
    """Bound on |dalpha_gpu - dalpha_ref| for the oracle's DalphaScale ``scale``; ``factor``
    scales every summand (a chain-rule factor applied to dalpha, e.g. d alpha / d theta)."""
    return factor * (DALPHA_C[dtype] * scale.rss_entry + DALPHA_ACC * scale.sum_abs)


def dalpha_check(got: float, ref: float, scale, dtype: int, factor: float = 1.0, label: str = "dalpha") -> None:
    """Asserts the dalpha bound; prints the error relative to |ref| and to the bound."""
    err = abs(float(got) - float(ref))
    bound = dalpha_bound(scale, dtype, factor)
    say(f"  {label} {float(got):.7g} vs {float(ref):.7g}: |err|/|ref| {err / max(abs(ref), 1e-30):.2e}, "
        f"|err|/bound {err / max(bound, 1e-30):.3f}, bound/|ref| {bound / max(abs(ref), 1e-30):.2e}, "
        f"|err|/(2^-8 rss_entry) {err / max(2.0 ** -8 * factor * scale.rss_entry, 1e-30):.3f}")
    assert err <= bound, (got, ref, bound)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(x32: np.ndarray, dtype: int):
    """(torch tensor on cuda:0 in the workload dtype, fp64 array of the exact same values)."""
    import torch
    if dtype == F32:
        t = torch.from_numpy(np.ascontiguousarray(x32)).cuda()
        return t, x32.astype(np.float64)
    bits = f32_to_bf16_bits(x32)
    t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return t, bf16_bits_to_f32(bits).astype(np.float64)


def inputs(seed: int, shape, dtype: int, with_dout: bool = False):
    arrs = normal_inputs(seed, shape, with_dout=with_dout)
    return [to_device(a, dtype) for a in arrs]


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def grad_excess(got, ref, dtype: int) -> float:
    """max over elements of |got - ref| - REL_ULP*|ref|; passes when <= TOL[dtype]."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.size(got):
        return 0.0
    return float(np.max(np.abs(got - ref) - REL_ULP[dtype] * np.abs(ref)))


def maxabs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64)))) if np.size(a) else 0.0
