"""The no-alloc backward (fib_sparse_attn_bwd_noalloc, workspace in the library's fixed
scratch) against the backward with a caller workspace (fib_sparse_attn_bwd), through the C
ABI: bit-identical gradients and dalpha (the same kernels on the same inputs), on two calls in
a row on one GPU, the second with a smaller input, so that the scratch keeps the first
call's contents when the second runs; integer and interpolated offsets, the bf16 ring kernels
and the fp32 general kernels.
"""
import numpy as np
import pytest
import torch

import fibonacci_offset_dilated_amd as F
from fibonacci_offset_dilated_amd.workloads import BF16, F32, FIB_BASE, INT, INTERP
from gpu_util import inputs, say

pytestmark = pytest.mark.gpu

# (B, H, N, W, alpha, dtype): a larger call, then a smaller one
PAIRS = [
    ((2, 4, 3000, 12, 1.37, BF16), (1, 2, 700, 12, 1.04, BF16)),
    ((1, 3, 2500, 12, 1.5, BF16), (1, 1, 300, 6, 0.77, BF16)),
    ((1, 2, 1200, 12, 1.21, F32), (1, 1, 500, 12, 0.93, F32)),
]


def _grads(shape, mode, seed):
    B, H, N, W, alpha, dtype = shape
    (q, _), (k, _), (v, _), (do, _) = inputs(seed, (B, H, N, 64), dtype, with_dout=True)
    a = np.float32(alpha)
    o, lse = F.fwd(q, k, v, W, a, FIB_BASE, 10000.0, mode)
    ref = F.bwd(q, k, v, o, lse, do, W, a, FIB_BASE, 10000.0, mode)
    # the no-alloc call writes into preallocated outputs that hold garbage beforehand
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    da = torch.full((1,), float("nan"), dtype=torch.float32, device=q.device)
    got = F.bwd_noalloc(q, k, v, o, lse, do, W, a, FIB_BASE, 10000.0, mode, dq=dq, dk=dk, dv=dv, dalpha=da)
    return ref, got


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("pair", PAIRS, ids=["bf16-a", "bf16-b", "f32"])
def test_noalloc_matches_workspace_backward(pair, mode):
    for step, shape in enumerate(pair):
        say("bwd_noalloc", shape, "mode", mode, "call", step)
        ref, got = _grads(shape, mode, 7100 + 10 * step + mode)
        torch.cuda.synchronize()
        for name, x, y in zip(("dQ", "dK", "dV", "dalpha"), ref, got):
            assert torch.equal(x, y), (name, shape, mode, step)


def test_noalloc_rejects_a_call_beyond_the_scratch():
    """The long-context interpolated backward needs more than the scratch: FibError, nothing
    launched (the inputs are never read, so empty tensors of the right shape suffice)."""
    q = torch.empty((1, 32, 131072, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 32, 131072), dtype=torch.float32, device="cuda")
    with pytest.raises(F.FibError, match="scratch"):
        F.bwd_noalloc(q, q, q, q, lse, q, 12, np.float32(1.5), FIB_BASE, 10000.0, INTERP, dq=q, dk=q, dv=q)
