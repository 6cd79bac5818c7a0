"""Pins of the oracle's schedules and offset tables (CPU only).

Checked against: a brute-force membership predicate over integer distances (a different
formulation of the rounding rule), hand-worked tables in tests/golden/hand_tables.txt, the
Fibonacci recurrence of the printed base, and exact rational facts about the schedules.
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from dense_reference import int_member, interp_virtuals
from fibonacci_offset_dilated_amd.workloads import FIB_BASE, POW2_BASE
from fibonacci_offset_dilated_amd.synthetic import random_alpha_grid

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_tables.txt")


def _f32_from_hex(h):
    return np.float32(struct.unpack(">f", bytes.fromhex(h))[0])


def _golden_rows():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, ah, W, mode, exp = (x.strip() for x in line.split("|"))
            rows.append((name, _f32_from_hex(ah), int(W), mode, exp))
    return rows


def test_fib_base_is_the_printed_sequence():
    # [FIB] Method: fib = [1, 2, 3, 5, ..., 987]: Fibonacci recurrence, distinct, last 987.
    assert FIB_BASE[:4] == (1, 2, 3, 5) and FIB_BASE[-1] == 987
    for a, b, c in zip(FIB_BASE, FIB_BASE[1:], FIB_BASE[2:]):
        assert c == a + b
    assert POW2_BASE == tuple(2 ** e for e in range(12))


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: r[0])
def test_hand_tables(row):
    name, alpha, W, mode, exp = row
    if mode == "int":
        want = [int(x) for x in exp.split(",")]
        assert O.int_offsets(alpha, FIB_BASE, W) == want
    else:
        want = []
        for t in exp.split(","):
            f, c, w = t.split(":")
            p, q = w.split("/")
            want.append((int(f), int(c), Fraction(int(p), int(q))))
        assert O.interp_entries(alpha, FIB_BASE, W) == want


def _alpha_grid():
    grid = list(O.schedule_linear(16)) + [np.float32(x) for x in (0.5, 1.0, 1.5, 0.7, 1.1, 1.3)]
    grid += list(random_alpha_grid(11, 40))
    # exact half-integer products: alpha = (2m+1)/(2f) for small f
    for f in (3, 5, 13, 21, 55):
        for m in (f // 2, f, f + 3):
            grid.append(np.float32((2 * m + 1) / (2 * f)))
    return grid


@pytest.mark.parametrize("W", [1, 6, 8, 10, 12, 20])
@pytest.mark.parametrize("base", [FIB_BASE, POW2_BASE], ids=["fib", "pow2"])
def test_int_table_vs_bruteforce_membership(W, base):
    for a in _alpha_grid():
        got = O.int_offsets(a, base, W)
        top = int(math.ceil(float(a) * max(base))) + 2
        want = [d for d in range(top) if int_member(d, a, base, W)]
        assert got == want, (a, W)


@pytest.mark.parametrize("W", [1, 6, 12])
@pytest.mark.parametrize("base", [FIB_BASE, POW2_BASE], ids=["fib", "pow2"])
def test_interp_entries_vs_definition(W, base):
    for a in _alpha_grid():
        got = O.interp_entries(a, base, W)
        want = interp_virtuals(a, base, W)
        assert [(f, c) for f, c, _ in got] == [(f, c) for f, c, _, _ in want]
        for (f, c, w), (_, _, _, wf) in zip(got, want):
            d = O.exact_alpha(a) * f
            assert c - 1 < d <= c and 0 <= w < 1 and w == c - d and float(w) == wf


def test_fp32_product_hazards_use_exact_product():
    # alpha_5 of the linear schedule is fp32(5/6); 21 * alpha is just below 17.5.
    lin = O.schedule_linear(16)
    a5 = lin[5]
    assert Fraction(float(a5)) * 21 < Fraction(35, 2)
    assert 17 in O.int_offsets(a5, FIB_BASE, 12) and 18 not in O.int_offsets(a5, FIB_BASE, 12)
    # the fp32 product would have tied at 17.5 and rounded to 18
    assert float(np.float32(a5) * np.float32(21)) == 17.5


def test_linear_schedule_exact_properties():
    lin = O.schedule_linear(16)
    assert lin[0] == np.float32(0.5) and lin[15] == np.float32(1.5)
    for l, a in enumerate(lin):
        exact = Fraction(1, 2) + Fraction(l, 15)
        ulp = Fraction(float(np.spacing(a)))
        assert abs(Fraction(float(a)) - exact) <= ulp / 2
    assert all(b > a for a, b in zip(lin, lin[1:]))


def test_coprime_schedule_is_permutation_and_involution():
    lin = O.schedule_linear(16)
    cop = O.schedule_coprime(16)
    assert sorted(cop) == sorted(lin)
    order = [(7 * l) % 16 for l in range(16)]
    assert order == [0, 7, 14, 5, 12, 3, 10, 1, 8, 15, 6, 13, 4, 11, 2, 9]
    assert all(order[order[l]] == l for l in range(16))
    assert [cop[l] for l in range(16)] == [lin[o] for o in order]
    # adjacent layers of the coprime order differ by at least 3 ramp steps (the pages' aim:
    # large spacing differences between neighbouring layers)
    assert min(abs(order[l + 1] - order[l]) for l in range(15)) >= 3


def test_table_errors():
    with pytest.raises(ValueError):
        O.int_offsets(1.0, [], 12)
    with pytest.raises(ValueError):
        O.int_offsets(1.0, [1, 1, 2], 12)
    with pytest.raises(ValueError):
        O.int_offsets(float("nan"), FIB_BASE, 12)


def test_index_set_cardinality_closed_form():
    # |S_i| = min(W, i + 1) + #{r in R : r <= i} in integer mode
    for a in (np.float32(1.0), O.schedule_linear(16)[3], np.float32(1.5)):
        for W in (1, 6, 12):
            R = O.int_offsets(a, FIB_BASE, W)
            ids = O.index_sets(1500, W, a, FIB_BASE, O.INT)
            for i in (0, 1, 5, 11, 12, 13, 100, 987, 1499):
                n = int((ids[i] >= 0).sum())
                assert n == min(W, i + 1) + sum(1 for r in R if r <= i)
                assert len(set(ids[i][ids[i] >= 0].tolist())) == n


# ---- index_sets, cell by cell, against sets built without the oracle ----------------------

def _int_offsets_brute(alpha, base, W):
    """Every integer distance that int_member accepts, ascending (searched up to beyond the
    largest product alpha * f, where no rounding can reach)."""
    top = int(float(np.float32(alpha)) * max(base)) + 2
    return [d for d in range(W, top + 1) if int_member(d, alpha, base, W)]


def _expected_int_rows(N, W, alpha, base):
    """[N, W + |R|]: window key i - s in column s (s <= i), then the keys at the brute-force
    distances in ascending distance order (each present when the distance is <= i)."""
    offs = _int_offsets_brute(alpha, base, W)
    out = -np.ones((N, W + len(offs)), dtype=np.int64)
    for i in range(N):
        win = list(range(i, max(-1, i - W), -1))  # keys i, i - 1, ... down to i - W + 1 and >= 0
        out[i, :len(win)] = win
        for e, d in enumerate(offs):
            if d <= i:
                out[i, W + e] = i - d
    return out


def _expected_interp_rows(N, W, alpha, base):
    """[N, W + n]: window keys as above, then per kept base entry (base order) the lower row
    of its interpolated pair, i - c with c the smallest integer >= alpha f (interp_virtuals'
    lo distance), present when c <= i."""
    virt = interp_virtuals(alpha, base, W)
    out = -np.ones((N, W + len(virt)), dtype=np.int64)
    for i in range(N):
        win = list(range(i, max(-1, i - W), -1))  # keys i, i - 1, ... down to i - W + 1 and >= 0
        out[i, :len(win)] = win
        for e, (_, c, c_hi, _) in enumerate(virt):
            assert c_hi == c - 1  # the upper row is the next row, i - c + 1
            if c <= i:
                out[i, W + e] = i - c
    return out


INDEX_CASES = [
    # (N, W, alpha, base): ties at 1.5 (55 -> 82.5, 987 -> 1480.5), W = 1, a window wider
    # than the sequence start, the power-of-two base, alpha at both ends of the range
    (1600, 12, np.float32(1.5), FIB_BASE),
    (400, 1, np.float32(1.0), FIB_BASE),
    (300, 12, O.schedule_linear(16)[5], FIB_BASE),
    (700, 6, np.float32(0.5), FIB_BASE),
    (2100, 12, np.float32(0.93), POW2_BASE),
    (40, 16, np.float32(1.37), FIB_BASE),
    (1, 12, np.float32(1.0), FIB_BASE),
]


@pytest.mark.parametrize("case", INDEX_CASES, ids=[f"N{c[0]}W{c[1]}a{float(c[2]):.4g}n{len(c[3])}" for c in INDEX_CASES])
def test_index_sets_int_cell_by_cell(case):
    N, W, a, base = case
    got = O.index_sets(N, W, a, base, O.INT)
    exp = _expected_int_rows(N, W, a, base)
    assert got.shape == exp.shape
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("case", INDEX_CASES, ids=[f"N{c[0]}W{c[1]}a{float(c[2]):.4g}n{len(c[3])}" for c in INDEX_CASES])
def test_index_sets_interp_cell_by_cell(case):
    N, W, a, base = case
    got = O.index_sets(N, W, a, base, O.INTERP)
    exp = _expected_interp_rows(N, W, a, base)
    assert got.shape == exp.shape
    assert np.array_equal(got, exp)


def test_index_sets_int_rows_are_the_brute_force_mask():
    """Integer mode: the set of rows in each query's row of index_sets equals the row of the
    brute-force mask M[i, j] = 0 <= j <= i and (i - j < W or i - j attended)."""
    from dense_reference import int_mask
    for N, W, a in ((260, 12, np.float32(1.3)), (150, 6, np.float32(0.5)), (90, 1, np.float32(1.0))):
        ids = O.index_sets(N, W, a, FIB_BASE, O.INT)
        M = int_mask(N, W, a, FIB_BASE)
        for i in range(N):
            assert set(ids[i][ids[i] >= 0].tolist()) == set(np.nonzero(M[i])[0].tolist())
