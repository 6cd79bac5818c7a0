"""GPU parity of the dense causal LSE (MFMA) and the dropped-attention-mass diagnostic
against the CPU oracle, via the C ABI.

Bounds: dense LSE within the bf16 LSE bound 2e-2 (rotated q and k are rounded to bf16 for the
MFMA, for fp32 inputs too; products accumulate in fp32). The dropped mass 1 - exp(lse_s -
lse_d) moves by at most (1 - dropped) |d lse_s - d lse_d| <= 2 x 2e-2, so its bound is 4e-2.
"""
import os

import numpy as np
import pytest
import torch

import fibonacci_offset_dilated_amd as F
import oracle as O
from fibonacci_offset_dilated_amd.workloads import BF16, F32, FIB_BASE, POW2_BASE
from gpu_util import TOL, host, inputs, maxabs, say

pytestmark = pytest.mark.gpu
TOL_DROPPED = 4e-2

LSE_CASES = [
    # (B, H, N, dtype)
    (1, 1, 1, BF16),
    (1, 2, 100, BF16),
    (2, 2, 1000, BF16),      # ragged: not a multiple of the 128-query or 64-key tiles
    (1, 3, 257, F32),
    (1, 2, 4096, BF16),      # the pages' evaluation length
    (1, 1, 128, BF16),
    (1, 1, 129, BF16),
]


@pytest.mark.parametrize("case", LSE_CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}-{'bf16' if c[3] else 'f32'}"
                                                 for c in LSE_CASES])
def test_dense_lse(case):
    B, H, N, dtype = case
    say("dense lse", case)
    (q, q64), (k, k64), _ = inputs(7700 + N, (B, H, N, 64), dtype)
    lse = F.dense_lse(q, k)
    torch.cuda.synchronize()
    ref = O.dense_causal_lse(q64, k64)
    e = maxabs(host(lse), ref)
    say(f"  max err {e:.3e}")
    assert e <= TOL[BF16]


DM_CASES = [
    # (B, H, N, W, alpha, base)
    (1, 2, 1024, 12, 1.0, FIB_BASE),
    (1, 2, 1024, 12, 1.0, POW2_BASE),
    (1, 2, 4096, 12, 1.5, FIB_BASE),
    (1, 2, 4096, 12, 1.0, POW2_BASE),
    (2, 1, 700, 6, 0.7, FIB_BASE),
    (1, 1, 300, 300, 1.0, FIB_BASE),      # W >= N: nothing is dropped
]


@pytest.mark.parametrize("case", DM_CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}W{c[3]}a{c[4]}n{len(c[5])}" for c in DM_CASES])
def test_dropped_mass(case):
    B, H, N, W, alpha, base = case
    say("dropped mass", case)
    (q, q64), (k, k64), (v, _) = inputs(7800 + N + W, (B, H, N, 64), BF16)
    a = np.float32(alpha)
    dm = F.dropped_mass(q, k, v, W, a, base)
    torch.cuda.synchronize()
    ref = O.dropped_mass(q64, k64, W, a, base)
    e = maxabs(host(dm), ref)
    say(f"  max err {e:.3e}; mean dropped {float(np.mean(ref)):.4f} (gpu {float(host(dm).mean()):.4f})")
    assert e <= TOL_DROPPED
    if W >= N:
        assert float(np.max(np.abs(host(dm)))) <= TOL_DROPPED


def test_dense_lse_rejects_bad_arguments():
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    L = F.lib()
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    lse = torch.empty((1, 1, 8), dtype=torch.float32, device="cuda")
    import ctypes
    assert L.fib_dense_causal_lse(q.data_ptr(), q.data_ptr(), lse.data_ptr(), 1, 1, 8, 64, 1,
                                  ctypes.c_float(10000.0), ws.data_ptr(), 16, None) == -11
