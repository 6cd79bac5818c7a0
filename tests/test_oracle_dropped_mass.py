"""Pins of the oracle's dense causal LSE and dropped-attention-mass diagnostic.

The diagnostic is the attention-gap measure of "SSA: Sparse Sparse Attention" (arXiv
2511.20102, gist.science Korean summary, 1. Problem definition, item 1): the weight that full
attention gives to keys outside the sparse set. Pins, each independent of the oracle's own
matmul-and-mask code:
  * zero queries give uniform attention over keys 0..i: LSE = log(i + 1) and the dropped mass
    is 1 - |S_i| / (i + 1), with |S_i| counted by hand from the pages' rules;
  * W >= N makes the sparse set the whole causal prefix: dropped mass 0, and the dense LSE
    equals the sparse oracle forward's LSE (a gather over the index set, another code path);
  * per-pair brute force with relative rotations <R_(i-j) q_i, k_j> (catches a transposed
    product or a mask off by one);
  * 0 <= dropped <= 1, and dropped = 0 for queries inside the window.
"""
import math

import numpy as np
import pytest

import oracle as O

FIB = (1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987)


def test_uniform_attention_closed_form():
    # q = 0: every logit is 0, so attention is uniform over the causal prefix
    N, D = 10, 8
    rng = np.random.default_rng(1)
    q = np.zeros((N, D))
    k = rng.standard_normal((N, D))
    lse = O.dense_causal_lse(q, k)
    assert np.allclose(lse, np.log(np.arange(1, N + 1)), atol=1e-14, rtol=0)
    # W = 2, alpha = 1, base (1, 2, 3, 5, 8): offsets 2, 3, 5, 8 (1 < W is dropped).
    # Query 9 attends {9, 8} + {7, 6, 4, 1} = 6 of its 10 keys; query 4 attends {4, 3} +
    # {2, 1} = 4 of 5 (offset 5 and 8 exceed i); query 1 attends {1, 0} = all.
    dm = O.dropped_mass(q, k, 2, 1.0, (1, 2, 3, 5, 8))
    assert abs(dm[9] - (1 - 6 / 10)) < 1e-14
    assert abs(dm[4] - (1 - 4 / 5)) < 1e-14
    assert abs(dm[1]) < 1e-14
    # query 7: {7, 6} + {5, 4, 2} (offsets 2, 3, 5; 8 > 7) = 5 of 8
    assert abs(dm[7] - (1 - 5 / 8)) < 1e-14


def test_uniform_attention_collapsed_offsets():
    # integer offsets that round to the same distance count once: alpha = 0.5 on base
    # (1, 2, 3, 4, 5, 6): 0.5 -> 0, 1, 1.5 -> 2, 2, 2.5 -> 2, 3; with W = 1 the set is {1, 2, 3}
    N = 6
    q = np.zeros((N, 4))
    k = np.ones((N, 4))
    dm = O.dropped_mass(q, k, 1, 0.5, (1, 2, 3, 4, 5, 6))
    # query 5: {5} + {4, 3, 2} = 4 of 6
    assert abs(dm[5] - (1 - 4 / 6)) < 1e-14


def test_full_window_drops_nothing_and_matches_sparse_lse():
    rng = np.random.default_rng(2)
    N, D = 40, 16
    q, k, v = (rng.standard_normal((1, 1, N, D)) for _ in range(3))
    dm = O.dropped_mass(q, k, N, 1.0, FIB)
    assert np.max(np.abs(dm)) < 1e-12
    lse_dense = O.dense_causal_lse(q, k)
    _, lse_sparse = O.forward(q, k, v, N, 1.0, FIB, 10000.0, O.INT)
    assert np.max(np.abs(lse_dense - lse_sparse)) < 1e-12


def test_dense_lse_brute_force_relative_rotation():
    rng = np.random.default_rng(3)
    N, D, theta = 17, 8, 500.0
    q = rng.standard_normal((N, D))
    k = rng.standard_normal((N, D))
    got = O.dense_causal_lse(q, k, theta)
    for i in range(N):
        logits = []
        for j in range(i + 1):
            # <R_i q, R_j k> = <R_(i-j) q, k>: rotate q alone by the relative position
            qi = O.rope(q[i:i + 1], theta, positions=[i - j])[0]
            logits.append(float(np.dot(qi, k[j])) / math.sqrt(D))
        m = max(logits)
        want = m + math.log(sum(math.exp(x - m) for x in logits))
        assert abs(got[i] - want) < 1e-12


@pytest.mark.parametrize("base,W,alpha", [(FIB, 12, 1.0), (tuple(2 ** e for e in range(12)), 12, 1.0),
                                          (FIB, 6, 1.5)])
def test_dropped_mass_range_and_window(base, W, alpha):
    rng = np.random.default_rng(4)
    N, D = 300, 64
    q = rng.standard_normal((N, D))
    k = rng.standard_normal((N, D))
    dm = O.dropped_mass(q, k, W, alpha, base)
    assert np.all(dm >= -1e-12) and np.all(dm <= 1 + 1e-12)
    assert np.max(np.abs(dm[:W])) < 1e-12  # the window covers every key of the first W queries
    # a wider window drops no more mass
    dm_w = O.dropped_mass(q, k, W + 8, alpha, base)
    assert np.all(dm_w <= dm + 1e-12)
