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
# bound on dalpha, relative to the sum over queries of |query's contribution| (the oracle's
# dalpha_abs): dalpha is a sum of per-query terms that can cancel, and each term carries the
# relative error of the forward's logits; without cancellation this is a plain relative bound
TOL_DALPHA = {F32: 1e-4, BF16: 1e-2}


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
