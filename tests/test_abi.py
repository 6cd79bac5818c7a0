"""Host-side tests of the C ABI (CPU only, no kernel launches).

The library loads and exports every function include/fibattn.h declares; the host offset
table and schedules equal the oracle's bit for bit; every argument error is reported before
anything is launched (the fake device pointers used here are never dereferenced because
validation fails first).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import fibonacci_offset_dilated_amd as F
import oracle as O
from fibonacci_offset_dilated_amd import _lib
from fibonacci_offset_dilated_amd.synthetic import random_alpha_grid
from fibonacci_offset_dilated_amd.workloads import FIB_BASE, POW2_BASE

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fibattn.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(fib_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 7
    L = F.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SYMBOLS)


def test_status_strings():
    for st in range(0, -16, -1):
        assert F.status_string(st) and F.status_string(st) != "unknown status"
    assert F.status_string(-99) == "unknown status"


def _grid():
    g = list(O.schedule_linear(16)) + list(random_alpha_grid(5, 30))
    g += [np.float32(x) for x in (0.5, 1.0, 1.5, 2.0, 0.013, 7.25)]
    return g


@pytest.mark.parametrize("W", [1, 6, 8, 10, 12, 16, 40])
@pytest.mark.parametrize("base", [FIB_BASE, POW2_BASE], ids=["fib", "pow2"])
def test_host_table_matches_oracle(W, base):
    for a in _grid():
        dist, w, f = F.offset_table(a, base, W, F.INT)
        assert dist == O.int_offsets(a, base, W), (a, W)
        assert all(x == 0 for x in w) and all(x == 0 for x in f)
        dist, w, f = F.offset_table(a, base, W, F.INTERP)
        ent = O.interp_entries(a, base, W)
        assert dist == [c for _, c, _ in ent]
        assert f == [ff for ff, _, _ in ent]
        # the kernels get w rounded to fp32 (nearest); the oracle keeps it exact
        assert [np.float32(x) for x in w] == [O.f32_nearest(ww) for _, _, ww in ent]


def test_schedules_match_oracle():
    for L in range(2, 41):
        lib_lin = [F.schedule_alpha(F.SCHED_LINEAR, l, L) for l in range(L)]
        assert lib_lin == list(O.schedule_linear(L)), L
        if L % 7:
            lib_cop = [F.schedule_alpha(F.SCHED_COPRIME, l, L) for l in range(L)]
            assert lib_cop == list(O.schedule_coprime(L)), L
    assert F.schedule_alpha(F.SCHED_FIXED, 3, 16) == np.float32(1.0)


@pytest.mark.parametrize("args", [(9, 0, 16), (F.SCHED_LINEAR, 16, 16), (F.SCHED_LINEAR, 0, 1),
                                  (F.SCHED_COPRIME, 0, 14), (F.SCHED_LINEAR, -1, 16)])
def test_schedule_errors(args):
    with pytest.raises(F.FibError) as ei:
        F.schedule_alpha(*args)
    assert ei.value.status == -13


def _fwd_raw(q=16, k=16, v=16, o=16, lse=0, B=1, H=1, N=8, D=64, dtype=1, W=12, alpha=1.0,
             base=FIB_BASE, theta=10000.0, mode=0):
    b = (ctypes.c_int32 * max(1, len(base)))(*base)
    return F.lib().fib_sparse_attn_fwd(q, k, v, o, lse, B, H, N, D, dtype, W, ctypes.c_float(alpha), b,
                                       len(base), ctypes.c_float(theta), mode, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(o=None), -1),
    (dict(B=0), -2), (dict(N=0), -2), (dict(H=-1), -2), (dict(N=1 << 32), -2),
    (dict(D=128), -3), (dict(D=63), -3),
    (dict(dtype=2), -4),
    (dict(W=0), -5),
    (dict(alpha=0.0), -6), (dict(alpha=-1.0), -6), (dict(alpha=float("inf")), -6), (dict(alpha=float("nan")), -6),
    (dict(base=()), -7), (dict(base=(1, 1, 2)), -7), (dict(base=(0, 1)), -7), (dict(base=(1, 1 << 25)), -7),
    (dict(base=tuple(range(1, 34))), -7),
    (dict(theta=0.0), -8), (dict(theta=float("nan")), -8),
    (dict(mode=2), -9),
    (dict(q=0x1008), -10), (dict(lse=0x1002), -10),
])
def test_fwd_argument_errors(kw, status):
    assert _fwd_raw(**kw) == status


def test_decode_argument_errors():
    L = F.lib()
    b = (ctypes.c_int32 * 15)(*FIB_BASE)
    p = 16

    def call(q=p, kc=p, o=p, lse=0, B=1, N=8, D=64, dtype=1, W=12, alpha=1.0, mode=0, nb=15):
        return L.fib_sparse_attn_decode(q, kc, p, o, lse, B, 1, N, D, dtype, W, ctypes.c_float(alpha), b, nb,
                                        ctypes.c_float(10000.0), mode, None)
    assert call(q=None) == -1 and call(kc=None) == -1 and call(o=None) == -1
    assert call(B=0) == -2 and call(N=0) == -2
    assert call(D=32) == -3
    assert call(dtype=5) == -4
    assert call(W=0) == -5
    assert call(alpha=float("nan")) == -6
    assert call(nb=0) == -7
    assert call(mode=3) == -9
    assert call(o=0x1004) == -10 and call(lse=0x1001) == -10


def test_device_alpha_argument_errors():
    L = F.lib()
    b = (ctypes.c_int32 * 15)(*FIB_BASE)
    p = 16
    need = F.plan_bytes()
    assert need > 0

    def fwd(alpha=p, lo=0.5, hi=1.5, plan=p, nbytes=need):
        return L.fib_sparse_attn_fwd_dev(p, p, p, p, None, 1, 1, 8, 64, 1, 12, alpha, ctypes.c_float(lo),
                                         ctypes.c_float(hi), b, 15, ctypes.c_float(10000.0), 1, plan, nbytes, None)
    assert fwd(alpha=None) == -1 and fwd(plan=None) == -1
    assert fwd(lo=0.0) == -6 and fwd(lo=1.6) == -6 and fwd(hi=float("inf")) == -6
    assert fwd(alpha=0x1002) == -10 and fwd(plan=0x1008) == -10
    assert fwd(nbytes=need - 1) == -11

    def bwd(alpha=p, plan=p, nbytes=need, ws=p, ws_bytes=1 << 40):
        return L.fib_sparse_attn_bwd_dev(p, p, p, p, p, p, p, p, p, p, 1, 1, 8, 64, 1, 12, alpha, ctypes.c_float(0.5),
                                         ctypes.c_float(1.5), b, 15, ctypes.c_float(10000.0), 1, ws, ws_bytes, plan,
                                         nbytes, None)
    assert bwd(alpha=None) == -1 and bwd(ws=None) == -11 and bwd(nbytes=3) == -11
    assert L.fib_sparse_attn_decode_dev(p, p, p, p, None, 1, 1, 8, 64, 1, 12, None, ctypes.c_float(0.5),
                                        ctypes.c_float(1.5), b, 15, ctypes.c_float(10000.0), 0, p, need, None) == -1


def test_layers_argument_errors():
    L = F.lib()
    b = (ctypes.c_int32 * 15)(*FIB_BASE)
    p = 16
    need = F.layers_plan_bytes(4)
    assert need == 4 * F.plan_bytes()
    assert F.layers_plan_bytes(0) == 0 and F.layers_plan_bytes(257) == 0 and F.layers_plan_bytes(256) > 0
    alphas = (ctypes.c_float * 4)(0.5, 0.8, 1.2, 1.5)

    def fwd(nl=4, alpha=alphas, plan=p, nbytes=need, B=1):
        return L.fib_sparse_attn_fwd_layers(p, p, p, p, None, nl, B, 1, 8, 64, 1, 12, alpha, b, 15,
                                            ctypes.c_float(10000.0), 0, plan, nbytes, None)
    assert fwd(alpha=None) == -1 and fwd(plan=None) == -1
    assert fwd(nl=0) == -2 and fwd(nl=257) == -2 and fwd(B=0) == -2
    assert fwd(nbytes=need - 1) == -11 and fwd(plan=0x1008) == -10
    bad = (ctypes.c_float * 4)(0.5, float("nan"), 1.2, 1.5)
    assert fwd(alpha=bad) == -6
    neg = (ctypes.c_float * 4)(0.5, 0.8, -1.0, 1.5)
    assert fwd(alpha=neg) == -6

    def fwd_dev(alpha=p, lo=0.5, hi=1.5, nbytes=need):
        return L.fib_sparse_attn_fwd_layers_dev(p, p, p, p, None, 4, 1, 1, 8, 64, 1, 12, alpha, ctypes.c_float(lo),
                                                ctypes.c_float(hi), b, 15, ctypes.c_float(10000.0), 1, p, nbytes,
                                                None)
    assert fwd_dev(alpha=None) == -1 and fwd_dev(lo=2.0) == -6 and fwd_dev(nbytes=need - 1) == -11

    def bwd(ws=p, ws_bytes=1 << 40, nbytes=need, alpha=alphas):
        return L.fib_sparse_attn_bwd_layers(p, p, p, p, p, p, p, p, p, p, 4, 1, 1, 8, 64, 1, 12, alpha, b, 15,
                                            ctypes.c_float(10000.0), 1, ws, ws_bytes, p, nbytes, None)
    assert bwd(alpha=None) == -1 and bwd(ws=None) == -11 and bwd(nbytes=need - 1) == -11
    # the workspace of L layers is the single-layer size at L * B batches, for the largest alpha
    ws_need = F.bwd_workspace_size(4, 1, 8, 64, F.BF16, F.INTERP, 12, 1.5, FIB_BASE)
    assert 0 < ws_need < F.bwd_workspace_size(4, 1, 8, 64, F.BF16, F.INTERP)
    assert bwd(ws_bytes=ws_need - 1) == -11
    assert L.fib_sparse_attn_bwd_layers_dev(p, p, p, p, p, p, p, p, p, p, 4, 1, 1, 8, 64, 1, 12, None,
                                            ctypes.c_float(0.5), ctypes.c_float(1.5), b, 15, ctypes.c_float(10000.0),
                                            1, p, 1 << 40, p, need, None) == -1


def test_dense_lse_argument_errors():
    L = F.lib()
    p = 16
    need = L.fib_dense_lse_workspace_size(1, 2, 100, 64, 1)
    assert need == 2 * 2 * 100 * 64 * 2
    assert L.fib_dense_lse_workspace_size(1, 2, 100, 32, 1) == 0

    def call(q=p, lse=p, ws=p, ws_bytes=need, theta=10000.0, D=64, dtype=1):
        return L.fib_dense_causal_lse(q, p, lse, 1, 2, 100, D, dtype, ctypes.c_float(theta), ws, ws_bytes, None)
    assert call(q=None) == -1 and call(lse=None) == -1
    assert call(ws=None) == -11 and call(ws_bytes=need - 1) == -11
    assert call(theta=0.0) == -8 and call(D=32) == -3 and call(dtype=7) == -4
    assert call(q=0x1008) == -10
    assert L.fib_sparse_attn_dropped_mass(None, p, p, 10, None) == -1
    assert L.fib_sparse_attn_dropped_mass(p, p, p, 0, None) == -2
    assert L.fib_sparse_attn_dropped_mass(p, 0x1002, p, 10, None) == -10


def test_bwd_argument_errors():
    L = F.lib()
    b = (ctypes.c_int32 * 15)(*FIB_BASE)
    p = 16

    def call(ws=p, ws_bytes=1 << 40, lse=p, mode=1, dalpha=p, dq=p):
        return L.fib_sparse_attn_bwd(p, p, p, p, p, lse, dq, p, p, dalpha, 1, 1, 8, 64, 1, 12,
                                     ctypes.c_float(1.0), b, 15, ctypes.c_float(10000.0), mode, ws, ws_bytes, None)
    assert call(lse=None) == -1
    assert call(dq=None) == -1
    assert call(mode=5) == -9
    assert call(ws=None) == -11
    assert call(ws_bytes=3) == -11
    assert call(dalpha=0x1002) == -10
    need = F.bwd_workspace_size(1, 1, 8, 64, F.BF16, F.INTERP, 12, 1.0, FIB_BASE)
    assert need > 0 and call(ws_bytes=need - 1) == -11


def test_workspace_size():
    big = F.bwd_workspace_size(1, 32, 131072, 64, F.BF16, F.INTERP)
    assert big >= 32 * 131072 * 4 * 32  # one 32-bit word per row and possible entry (32)
    assert F.bwd_workspace_size(0, 1, 8, 64, F.BF16, F.INT) == 0
    assert F.bwd_workspace_size(1, 1, 8, 32, F.BF16, F.INT) == 0
    # for a known base and alpha: the entries alpha * f >= W only (11 at alpha 1.5, W 12)
    # (interpolated bf16 calls also hold the rotated q and k rows: 2 x 64 bf16 per row)
    exact = F.bwd_workspace_size(1, 32, 131072, 64, F.BF16, F.INTERP, 12, 1.5, FIB_BASE)
    int_ws = F.bwd_workspace_size(1, 32, 131072, 64, F.BF16, F.INT)
    assert exact - int_ws == 32 * 131072 * (2 * 64 * 2 + 4 * 11)
    assert F.bwd_workspace_size(1, 32, 131072, 64, F.BF16, F.INT, 12, 1.5, FIB_BASE) == int_ws
    assert big - int_ws == 32 * 131072 * (2 * 64 * 2 + 4 * 32)
    assert int_ws == F.bwd_workspace_size(1, 32, 131072, 64, F.F32, F.INT)
    # fp32 inputs use no (P, dS) words; bad arguments give 0
    assert F.bwd_workspace_size(1, 2, 100, 64, F.F32, F.INTERP, 12, 1.5, FIB_BASE) == \
        F.bwd_workspace_size(1, 2, 100, 64, F.F32, F.INT)
    assert F.bwd_workspace_size(1, 2, 100, 64, F.BF16, F.INTERP, 0, 1.5, FIB_BASE) == 0
    assert F.bwd_workspace_size(1, 2, 100, 64, F.BF16, F.INTERP, 12, float("nan"), FIB_BASE) == 0
    assert F.bwd_workspace_size(1, 2, 100, 64, F.BF16, F.INTERP, 12, 1.0, (3, 2)) == 0


def test_index_set_argument_errors():
    L = F.lib()
    b = (ctypes.c_int32 * 15)(*FIB_BASE)
    assert L.fib_sparse_attn_index_set(8, 12, ctypes.c_float(1.0), b, 15, 0, None, 22, None) == -1
    assert L.fib_sparse_attn_index_set(8, 12, ctypes.c_float(1.0), b, 15, 0, 16, 21, None) == -14
    assert L.fib_sparse_attn_index_set(0, 12, ctypes.c_float(1.0), b, 15, 0, 16, 22, None) == -2


def test_no_fallback_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libfibattn.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_bwd_noalloc_argument_errors():
    """The no-alloc backward reports argument errors like fib_sparse_attn_bwd and rejects a
    call whose workspace would exceed the fixed scratch, before anything is launched."""
    L = F.lib()
    b = (ctypes.c_int32 * 15)(*FIB_BASE)
    p = 16

    def call(B=1, H=1, N=8, mode=1, lse=p, dq=p, alpha=1.0, W=12, dtype=1, nb=15):
        return L.fib_sparse_attn_bwd_noalloc(p, p, p, p, p, lse, dq, p, p, p, B, H, N, 64, dtype, W,
                                             ctypes.c_float(alpha), b, nb, ctypes.c_float(10000.0), mode, None)
    assert call(lse=None) == -1 and call(dq=None) == -1
    assert call(mode=5) == -9 and call(W=0) == -5 and call(alpha=float("nan")) == -6
    assert call(B=0) == -2 and call(dtype=3) == -4 and call(nb=0) == -7
    # the long-context interpolated backward needs ~1.1 GB for the rotated rows and ~201 MB of
    # (P, dS) words: more than 64 MiB
    need = F.bwd_workspace_size(1, 32, 131072, 64, F.BF16, F.INTERP, 12, 1.5, FIB_BASE)
    assert need > F.NOALLOC_SCRATCH_BYTES
    assert call(B=1, H=32, N=131072, alpha=1.5) == -15
    # its integer-mode backward fits, and so does the interpolated one at the training shape
    assert F.bwd_workspace_size(1, 32, 131072, 64, F.BF16, F.INT, 12, 1.5, FIB_BASE) <= F.NOALLOC_SCRATCH_BYTES
    assert F.bwd_workspace_size(8, 8, 1024, 64, F.BF16, F.INTERP, 12, 1.05, FIB_BASE) <= F.NOALLOC_SCRATCH_BYTES
    assert "scratch" in F.status_string(-15)
