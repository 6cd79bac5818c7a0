"""GPU parity of the decode step (one query at the newest position of a K/V cache) against
the CPU oracle, via the C ABI.

The decode query of position N - 1 is row N - 1 of a seeded [B, H, N, D] draw of Q; its
oracle result is row N - 1 of the oracle forward over the cache. Bounds: max-abs error on O
and LSE within 1e-4 (fp32) / 2e-2 (bf16), as for the forward.
"""
import numpy as np
import pytest
import torch

import fibonacci_offset_dilated_amd as F
import oracle as O
from fibonacci_offset_dilated_amd.workloads import BF16, F32, FIB_BASE, INT, INTERP, POW2_BASE
from gpu_util import TOL, host, inputs, maxabs, say

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, N, W, alpha, base, dtype)
    (1, 1, 1, 12, 1.0, FIB_BASE, BF16),        # the query alone
    (2, 3, 2, 12, 1.0, FIB_BASE, BF16),
    (2, 4, 1000, 12, 1.5, FIB_BASE, BF16),
    (1, 8, 4096, 12, 1.0, FIB_BASE, BF16),     # the pages' evaluation length
    (3, 2, 5000, 40, 0.93, POW2_BASE, BF16),
    (1, 2, 300, 130, 1.0, FIB_BASE, BF16),     # more keys than the block's 64 quads
    (1, 1, 70000, 6, 1.37, FIB_BASE, BF16),
    (2, 2, 1700, 16, 1.0001, (1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 511, 512, 610), BF16),
    (2, 3, 1000, 12, 1.21, FIB_BASE, F32),
    (1, 2, 65, 1, 0.5, FIB_BASE, F32),
]


def run_case(case, mode):
    B, H, N, W, alpha, base, dtype = case
    a = np.float32(alpha)
    (q, q64), (k, k64), (v, v64) = inputs(7000 + N + W, (B, H, N, 64), dtype)
    qd = q[:, :, N - 1, :].contiguous()
    o, lse = F.decode(qd, k, v, W, a, base, 10000.0, mode)
    torch.cuda.synchronize()
    go, gl = host(o), host(lse)
    eo = el = 0.0
    for b in range(B):
        for h in range(H):
            ro, rl = O.forward_rows(q64[b, h], k64[b, h], v64[b, h], np.array([N - 1]), W, a, base, 10000.0, mode)
            eo = max(eo, maxabs(go[b, h], ro[0]))
            el = max(el, maxabs(gl[b, h], rl[0]))
    return eo, el, (q, k, v, o, lse, a)


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}W{c[3]}a{c[4]}n{len(c[5])}-{'bf16' if c[6] else 'f32'}"
                                             for c in CASES])
def test_decode_parity(case, mode):
    say("decode", case[:5], len(case[5]), "bf16" if case[6] else "f32", "mode", mode)
    eo, el, _ = run_case(case, mode)
    say(f"  max err O {eo:.3e} LSE {el:.3e}")
    assert eo <= TOL[case[6]] and el <= TOL[case[6]]


@pytest.mark.parametrize("mode", [INT, INTERP], ids=["int", "interp"])
def test_decode_matches_forward_last_row(mode):
    """The decode step and the full forward agree on row N - 1 (two kernels, same values)."""
    case = (2, 4, 3000, 12, 1.5, FIB_BASE, BF16)
    _, _, (q, k, v, o, lse, a) = run_case(case, mode)
    of, lf = F.fwd(q, k, v, 12, a, FIB_BASE, 10000.0, mode)
    torch.cuda.synchronize()
    d_o = maxabs(host(o), host(of[:, :, -1, :]))
    d_l = maxabs(host(lse), host(lf[:, :, -1]))
    say(f"decode vs forward row N-1: O {d_o:.3e} LSE {d_l:.3e}")
    assert d_o <= 2 * TOL[BF16] and d_l <= 2 * TOL[BF16]


def test_decode_rejects_bad_shapes():
    k = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        F.decode(torch.zeros((1, 2, 1, 64), dtype=torch.bfloat16, device="cuda"), k, k, 12, 1.0, FIB_BASE)
    with pytest.raises(ValueError):
        F.decode(torch.zeros((1, 2, 64), dtype=torch.float32, device="cuda"), k, k, 12, 1.0, FIB_BASE)
