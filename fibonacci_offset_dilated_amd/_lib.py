"""ctypes binding of libfibattn.so (the C ABI declared in include/fibattn.h).

Argument marshalling only: every step of the attention runs in the library's HIP kernels.
torch supplies device memory and the current HIP stream. The library must have been built
(``python -m fibonacci_offset_dilated_amd.build``); loading fails loudly otherwise, and there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfibattn.so")

FIB_OK = 0
F32, BF16 = 0, 1
INT, INTERP = 0, 1
SCHED_FIXED, SCHED_LINEAR, SCHED_COPRIME = 0, 1, 2
MAX_BASE = 32

_lib = None

# exported symbols and their ctypes signatures (mirrors include/fibattn.h)
_c = ctypes
_SIGS = {
    "fib_sparse_attn_fwd": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                       _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int,
                                       _c.c_int, _c.c_float, _c.c_void_p, _c.c_int, _c.c_float, _c.c_int,
                                       _c.c_void_p]),
    "fib_sparse_attn_bwd": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                       _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                       _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int,
                                       _c.c_int, _c.c_float, _c.c_void_p, _c.c_int, _c.c_float, _c.c_int,
                                       _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "fib_sparse_attn_decode": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                          _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int,
                                          _c.c_int, _c.c_float, _c.c_void_p, _c.c_int, _c.c_float, _c.c_int,
                                          _c.c_void_p]),
    "fib_sparse_attn_plan_bytes": (_c.c_size_t, []),
    "fib_sparse_attn_fwd_dev": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                           _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int,
                                           _c.c_int, _c.c_void_p, _c.c_float, _c.c_float, _c.c_void_p, _c.c_int,
                                           _c.c_float, _c.c_int, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "fib_sparse_attn_decode_dev": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                              _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int,
                                              _c.c_int, _c.c_void_p, _c.c_float, _c.c_float, _c.c_void_p, _c.c_int,
                                              _c.c_float, _c.c_int, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "fib_sparse_attn_bwd_dev": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                           _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                           _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int,
                                           _c.c_int, _c.c_void_p, _c.c_float, _c.c_float, _c.c_void_p, _c.c_int,
                                           _c.c_float, _c.c_int, _c.c_void_p, _c.c_size_t, _c.c_void_p, _c.c_size_t,
                                           _c.c_void_p]),
    "fib_sparse_attn_bwd_noalloc": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                               _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                               _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int,
                                               _c.c_int, _c.c_float, _c.c_void_p, _c.c_int, _c.c_float, _c.c_int,
                                               _c.c_void_p]),
    "fib_sparse_attn_bwd_workspace_size": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64,
                                                         _c.c_int, _c.c_int]),
    "fib_sparse_attn_bwd_workspace_size_for": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64,
                                                             _c.c_int, _c.c_int, _c.c_int, _c.c_float, _c.c_void_p,
                                                             _c.c_int]),
    "fib_sparse_attn_layers_plan_bytes": (_c.c_size_t, [_c.c_int64]),
    "fib_dense_lse_workspace_size": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int]),
    "fib_dense_causal_lse": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64,
                                        _c.c_int64, _c.c_int, _c.c_float, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "fib_sparse_attn_dropped_mass": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p]),
    "fib_sparse_attn_fwd_layers": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                              _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int,
                                              _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_float, _c.c_int,
                                              _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "fib_sparse_attn_decode_layers": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                                 _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64,
                                                 _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_float,
                                                 _c.c_int, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "fib_sparse_attn_decode_layers_dev": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                                     _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64,
                                                     _c.c_int64, _c.c_int, _c.c_int, _c.c_void_p, _c.c_float,
                                                     _c.c_float, _c.c_void_p, _c.c_int, _c.c_float, _c.c_int,
                                                     _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "fib_sparse_attn_fwd_layers_dev": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                                  _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64,
                                                  _c.c_int, _c.c_int, _c.c_void_p, _c.c_float, _c.c_float,
                                                  _c.c_void_p, _c.c_int, _c.c_float, _c.c_int, _c.c_void_p,
                                                  _c.c_size_t, _c.c_void_p]),
    "fib_sparse_attn_bwd_layers": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                              _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                              _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int,
                                              _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_float, _c.c_int,
                                              _c.c_void_p, _c.c_size_t, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "fib_sparse_attn_bwd_layers_dev": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                                  _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                                  _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64,
                                                  _c.c_int, _c.c_int, _c.c_void_p, _c.c_float, _c.c_float,
                                                  _c.c_void_p, _c.c_int, _c.c_float, _c.c_int, _c.c_void_p,
                                                  _c.c_size_t, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "fib_status_string": (_c.c_char_p, [_c.c_int]),
    "fib_sparse_attn_offset_table": (_c.c_int, [_c.c_float, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int,
                                                _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "fib_sparse_attn_index_set": (_c.c_int, [_c.c_int64, _c.c_int, _c.c_float, _c.c_void_p, _c.c_int,
                                             _c.c_int, _c.c_void_p, _c.c_int64, _c.c_void_p]),
    "fib_schedule_alpha": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_void_p]),
}
SYMBOLS = tuple(_SIGS)


class FibError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libfibattn.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m fibonacci_offset_dilated_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fib_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != FIB_OK:
        raise FibError(status, where)


_BASE_ARRAYS: dict = {}


def _base_array(base: Sequence[int]):
    """ctypes int32 copy of the base offsets (cached per distinct base: the library only
    reads it during a call)."""
    key = tuple(base)
    hit = _BASE_ARRAYS.get(key)
    if hit is None:
        arr = (ctypes.c_int32 * max(1, len(key)))(*[int(b) for b in key])
        if len(_BASE_ARRAYS) >= 64:
            _BASE_ARRAYS.clear()
        hit = _BASE_ARRAYS[key] = (arr, len(key))
    return hit


def schedule_alpha(kind: int, layer: int, n_layers: int) -> np.float32:
    out = ctypes.c_float()
    _check(lib().fib_schedule_alpha(int(kind), int(layer), int(n_layers), ctypes.byref(out)), "fib_schedule_alpha")
    return np.float32(out.value)


def offset_table(alpha, base: Sequence[int], W: int, mode: int):
    """The library's offset table: (dist, w, f) lists (see fib_sparse_attn_offset_table)."""
    b, n = _base_array(base)
    cap = max(1, n)
    dist = (ctypes.c_int32 * cap)()
    w = (ctypes.c_float * cap)()
    f = (ctypes.c_int32 * cap)()
    cnt = ctypes.c_int()
    _check(lib().fib_sparse_attn_offset_table(ctypes.c_float(float(np.float32(alpha))), b, n, int(W), int(mode),
                                              dist, w, f, ctypes.byref(cnt)), "fib_sparse_attn_offset_table")
    m = cnt.value
    return list(dist[:m]), [np.float32(x) for x in w[:m]], list(f[:m])


# ---- torch-facing wrappers ---------------------------------------------------------------

_TORCH = None


def _torch():
    global _TORCH
    if _TORCH is None:
        import torch
        _TORCH = torch
    return _TORCH


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _stream(stream):
    """hipStream_t of `stream`, or of the current device's current stream when None (read
    through torch's raw-stream query, which skips building a Stream object)."""
    torch = _torch()
    if stream is None:
        C = torch._C
        if hasattr(C, "_cuda_getCurrentRawStream"):
            return ctypes.c_void_p(C._cuda_getCurrentRawStream(C._cuda_getDevice()))
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(fn):
    """Runs a binding call with `stream` (when given) as torch's current stream, so that every
    tensor the binding allocates (outputs, workspace, plan, temporaries) belongs to that
    stream in torch's caching allocator: a temporary dropped on return is then reused only by
    later work on the same stream, never while the call's kernels may still use it."""
    import functools

    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, stream=None, **kw)
        with _torch().cuda.stream(stream):
            return fn(*args, stream=stream, **kw)

    return call


def _check_qkv(*ts):
    Tensor = _torch().Tensor
    ref = ts[0]
    if not isinstance(ref, Tensor) or ref.get_device() < 0:
        raise TypeError("tensors must be CUDA (HIP) tensors")
    shape, dtype, dev = ref.shape, ref.dtype, ref.get_device()
    if len(shape) != 4:
        raise ValueError("q, k, v (and o, dout, grads) must share shape [B, H, N, D], dtype and device")
    for t in ts:
        if not isinstance(t, Tensor) or t.get_device() < 0:
            raise TypeError("tensors must be CUDA (HIP) tensors")
        if t.shape != shape or t.dtype != dtype or t.get_device() != dev:
            raise ValueError("q, k, v (and o, dout, grads) must share shape [B, H, N, D], dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


@_on_stream
def fwd(q, k, v, W: int, alpha, base: Sequence[int], theta: float = 10000.0, mode: int = INT,
        out=None, lse=None, with_lse: bool = True, stream=None):
    """Sparse attention forward on the current stream; returns (O, LSE or None)."""
    torch = _torch()
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_qkv(q, out)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    b, n = _base_array(base)
    st = lib().fib_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, D, _dtype_code(q),
                                   int(W), ctypes.c_float(float(np.float32(alpha))), b, n,
                                   ctypes.c_float(float(theta)), int(mode), _stream(stream))
    _check(st, "fib_sparse_attn_fwd")
    return out, lse


@_on_stream
def decode(q, k_cache, v_cache, W: int, alpha, base: Sequence[int], theta: float = 10000.0, mode: int = INT,
           out=None, lse=None, with_lse: bool = True, stream=None):
    """One decode step: q [B, H, D] at position N - 1 of the caches [B, H, N, D]; returns
    (O [B, H, D], LSE [B, H] or None)."""
    torch = _torch()
    _check_qkv(k_cache, v_cache)
    B, H, N, D = k_cache.shape
    for t in (q, out):
        if t is None:
            continue
        if (not isinstance(t, torch.Tensor) or not t.is_cuda or t.shape != (B, H, D) or t.dtype != k_cache.dtype
                or t.device != k_cache.device or not t.is_contiguous()):
            raise ValueError("q and o must be contiguous [B, H, D] tensors of the caches' dtype and device")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    b, n = _base_array(base)
    st = lib().fib_sparse_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), B, H, N, D,
                                      _dtype_code(q), int(W), ctypes.c_float(float(np.float32(alpha))), b, n,
                                      ctypes.c_float(float(theta)), int(mode), _stream(stream))
    _check(st, "fib_sparse_attn_decode")
    return out, lse


def plan_bytes() -> int:
    """Device bytes of the plan buffer of the device-alpha calls."""
    return int(lib().fib_sparse_attn_plan_bytes())


def _alpha_dev(alpha, device):
    torch = _torch()
    if (not isinstance(alpha, torch.Tensor) or alpha.dtype != torch.float32 or alpha.numel() != 1
            or alpha.device != device):
        raise ValueError("alpha must be a one-element float32 tensor on the inputs' device")
    return alpha


def _plan_buffer(plan, device):
    torch = _torch()
    need = plan_bytes()
    if plan is None:
        plan = torch.empty(need, dtype=torch.uint8, device=device)
    if plan.numel() * plan.element_size() < need:
        raise ValueError("plan buffer too small")
    return plan


@_on_stream
def fwd_dev(q, k, v, W: int, alpha, alpha_range, base: Sequence[int], theta: float = 10000.0, mode: int = INT,
            out=None, lse=None, with_lse: bool = True, plan=None, stream=None):
    """Forward with alpha a one-element float32 device tensor (no host copy of alpha);
    alpha_range = (lo, hi) bounds it (the kernels clamp it into the range)."""
    torch = _torch()
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    alpha = _alpha_dev(alpha, q.device)
    plan = _plan_buffer(plan, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_qkv(q, out)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    b, n = _base_array(base)
    lo, hi = alpha_range
    st = lib().fib_sparse_attn_fwd_dev(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, D, _dtype_code(q),
                                       int(W), _ptr(alpha), ctypes.c_float(float(lo)), ctypes.c_float(float(hi)),
                                       b, n, ctypes.c_float(float(theta)), int(mode), _ptr(plan),
                                       plan.numel() * plan.element_size(), _stream(stream))
    _check(st, "fib_sparse_attn_fwd_dev")
    return out, lse


@_on_stream
def bwd_dev(q, k, v, o, lse, dout, W: int, alpha, alpha_range, base: Sequence[int], theta: float = 10000.0,
            mode: int = INT, dq=None, dk=None, dv=None, dalpha=None, workspace=None, want_dalpha: bool = True,
            plan=None, stream=None):
    """Backward with alpha in device memory (see fwd_dev); returns (dQ, dK, dV, dalpha [1] or None)."""
    torch = _torch()
    _check_qkv(q, k, v, o, dout)
    B, H, N, D = q.shape
    alpha = _alpha_dev(alpha, q.device)
    plan = _plan_buffer(plan, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check_qkv(q, dq, dk, dv)
    if dalpha is None and want_dalpha:
        dalpha = torch.empty(1, dtype=torch.float32, device=q.device)
    lo, hi = alpha_range
    need = bwd_workspace_size(B, H, N, D, _dtype_code(q), mode, W, hi, base)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    b, n = _base_array(base)
    st = lib().fib_sparse_attn_bwd_dev(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dalpha), B, H, N, D, _dtype_code(q),
                                       int(W), _ptr(alpha), ctypes.c_float(float(lo)), ctypes.c_float(float(hi)),
                                       b, n, ctypes.c_float(float(theta)), int(mode), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _ptr(plan),
                                       plan.numel() * plan.element_size(), _stream(stream))
    _check(st, "fib_sparse_attn_bwd_dev")
    return dq, dk, dv, dalpha


@_on_stream
def decode_dev(q, k_cache, v_cache, W: int, alpha, alpha_range, base: Sequence[int], theta: float = 10000.0,
               mode: int = INT, out=None, lse=None, with_lse: bool = True, plan=None, stream=None):
    """Decode step with alpha in device memory (see fwd_dev and decode)."""
    torch = _torch()
    _check_qkv(k_cache, v_cache)
    B, H, N, D = k_cache.shape
    for t in (q, out):
        if t is None:
            continue
        if (not isinstance(t, torch.Tensor) or not t.is_cuda or t.shape != (B, H, D) or t.dtype != k_cache.dtype
                or t.device != k_cache.device or not t.is_contiguous()):
            raise ValueError("q and o must be contiguous [B, H, D] tensors of the caches' dtype and device")
    alpha = _alpha_dev(alpha, q.device)
    plan = _plan_buffer(plan, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    b, n = _base_array(base)
    lo, hi = alpha_range
    st = lib().fib_sparse_attn_decode_dev(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), B, H, N, D,
                                          _dtype_code(q), int(W), _ptr(alpha), ctypes.c_float(float(lo)),
                                          ctypes.c_float(float(hi)), b, n, ctypes.c_float(float(theta)), int(mode),
                                          _ptr(plan), plan.numel() * plan.element_size(), _stream(stream))
    _check(st, "fib_sparse_attn_decode_dev")
    return out, lse


def layers_plan_bytes(n_layers: int) -> int:
    """Device bytes of the plan buffer of a call over n_layers layers (0 if out of range)."""
    return int(lib().fib_sparse_attn_layers_plan_bytes(int(n_layers)))


def _check_layers(*ts):
    torch = _torch()
    ref = ts[0]
    for t in ts:
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError("tensors must be CUDA (HIP) tensors")
        if t.dim() != 5 or t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("layer tensors must share shape [L, B, H, N, D], dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _layers_alpha(alpha, L, alpha_range, device):
    """(host float32 array or None, device tensor or None, lo, hi) of a call over L layers."""
    torch = _torch()
    if alpha_range is None:
        a = np.ascontiguousarray(np.asarray(alpha, dtype=np.float32).reshape(-1))
        if a.size != L:
            raise ValueError(f"alpha must hold {L} values (one per layer)")
        return a, None, 0.0, 0.0
    if (not isinstance(alpha, torch.Tensor) or alpha.dtype != torch.float32 or alpha.numel() != L
            or alpha.device != device or not alpha.is_contiguous()):
        raise ValueError(f"alpha must be a contiguous float32 tensor of {L} values on the inputs' device")
    return None, alpha, float(alpha_range[0]), float(alpha_range[1])


def _layers_plan(plan, L, device):
    torch = _torch()
    need = layers_plan_bytes(L)
    if need == 0:
        raise ValueError("layer count out of range")
    if plan is None:
        plan = torch.empty(need, dtype=torch.uint8, device=device)
    if plan.numel() * plan.element_size() < need:
        raise ValueError("plan buffer too small")
    return plan


@_on_stream
def fwd_layers(q, k, v, W: int, alpha, base: Sequence[int], theta: float = 10000.0, mode: int = INT,
               alpha_range=None, out=None, lse=None, with_lse: bool = True, plan=None, stream=None):
    """Forward of L layers in one call: q, k, v [L, B, H, N, D]; alpha: L host values, or
    (with alpha_range = (lo, hi)) a float32 device tensor of L values. Returns (O, LSE [L, B,
    H, N] or None)."""
    torch = _torch()
    _check_layers(q, k, v)
    L, B, H, N, D = q.shape
    ah, ad, lo, hi = _layers_alpha(alpha, L, alpha_range, q.device)
    plan = _layers_plan(plan, L, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_layers(q, out)
    if lse is None and with_lse:
        lse = torch.empty((L, B, H, N), dtype=torch.float32, device=q.device)
    b, n = _base_array(base)
    pb = plan.numel() * plan.element_size()
    if ad is None:
        st = lib().fib_sparse_attn_fwd_layers(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), L, B, H, N, D,
                                              _dtype_code(q), int(W), ah.ctypes.data_as(ctypes.c_void_p), b, n,
                                              ctypes.c_float(float(theta)), int(mode), _ptr(plan), pb,
                                              _stream(stream))
        _check(st, "fib_sparse_attn_fwd_layers")
    else:
        st = lib().fib_sparse_attn_fwd_layers_dev(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), L, B, H, N, D,
                                                  _dtype_code(q), int(W), _ptr(ad), ctypes.c_float(lo),
                                                  ctypes.c_float(hi), b, n, ctypes.c_float(float(theta)), int(mode),
                                                  _ptr(plan), pb, _stream(stream))
        _check(st, "fib_sparse_attn_fwd_layers_dev")
    return out, lse


@_on_stream
def decode_layers(q, k_cache, v_cache, W: int, alpha, base: Sequence[int], theta: float = 10000.0, mode: int = INT,
                  alpha_range=None, out=None, lse=None, with_lse: bool = True, plan=None, stream=None):
    """One decode step of L layers in one launch: q [L, B, H, D] at position N - 1 of the caches
    [L, B, H, N, D]; alpha as in fwd_layers. Returns (O [L, B, H, D], LSE [L, B, H] or None)."""
    torch = _torch()
    _check_layers(k_cache, v_cache)
    L, B, H, N, D = k_cache.shape
    for t in (q, out):
        if t is None:
            continue
        if (not isinstance(t, torch.Tensor) or not t.is_cuda or t.shape != (L, B, H, D)
                or t.dtype != k_cache.dtype or t.device != k_cache.device or not t.is_contiguous()):
            raise ValueError("q and o must be contiguous [L, B, H, D] tensors of the caches' dtype and device")
    ah, ad, lo, hi = _layers_alpha(alpha, L, alpha_range, q.device)
    plan = _layers_plan(plan, L, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((L, B, H), dtype=torch.float32, device=q.device)
    b, n = _base_array(base)
    pb = plan.numel() * plan.element_size()
    if ad is None:
        st = lib().fib_sparse_attn_decode_layers(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), L, B, H,
                                                 N, D, _dtype_code(q), int(W), ah.ctypes.data_as(ctypes.c_void_p), b,
                                                 n, ctypes.c_float(float(theta)), int(mode), _ptr(plan), pb,
                                                 _stream(stream))
        _check(st, "fib_sparse_attn_decode_layers")
    else:
        st = lib().fib_sparse_attn_decode_layers_dev(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), L,
                                                     B, H, N, D, _dtype_code(q), int(W), _ptr(ad), ctypes.c_float(lo),
                                                     ctypes.c_float(hi), b, n, ctypes.c_float(float(theta)),
                                                     int(mode), _ptr(plan), pb, _stream(stream))
        _check(st, "fib_sparse_attn_decode_layers_dev")
    return out, lse


@_on_stream
def bwd_layers(q, k, v, o, lse, dout, W: int, alpha, base: Sequence[int], theta: float = 10000.0, mode: int = INT,
               alpha_range=None, dq=None, dk=None, dv=None, dalpha=None, workspace=None, want_dalpha: bool = True,
               plan=None, stream=None):
    """Backward of L layers in one call (see fwd_layers); returns (dQ, dK, dV, dalpha [L] or None)."""
    torch = _torch()
    _check_layers(q, k, v, o, dout)
    L, B, H, N, D = q.shape
    ah, ad, lo, hi = _layers_alpha(alpha, L, alpha_range, q.device)
    plan = _layers_plan(plan, L, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check_layers(q, dq, dk, dv)
    if dalpha is None and want_dalpha:
        dalpha = torch.empty(L, dtype=torch.float32, device=q.device)
    need = bwd_workspace_size(L * B, H, N, D, _dtype_code(q), mode, W, hi if ad is not None else float(np.max(ah)),
                              base)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    b, n = _base_array(base)
    pb = plan.numel() * plan.element_size()
    wb = workspace.numel() * workspace.element_size()
    common = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dalpha),
              L, B, H, N, D, _dtype_code(q), int(W))
    if ad is None:
        st = lib().fib_sparse_attn_bwd_layers(*common, ah.ctypes.data_as(ctypes.c_void_p), b, n,
                                              ctypes.c_float(float(theta)), int(mode), _ptr(workspace), wb,
                                              _ptr(plan), pb, _stream(stream))
        _check(st, "fib_sparse_attn_bwd_layers")
    else:
        st = lib().fib_sparse_attn_bwd_layers_dev(*common, _ptr(ad), ctypes.c_float(lo), ctypes.c_float(hi), b, n,
                                                  ctypes.c_float(float(theta)), int(mode), _ptr(workspace), wb,
                                                  _ptr(plan), pb, _stream(stream))
        _check(st, "fib_sparse_attn_bwd_layers_dev")
    return dq, dk, dv, dalpha


@_on_stream
def dense_lse(q, k, theta: float = 10000.0, lse=None, workspace=None, stream=None):
    """LSE [B, H, N] of dense causal attention over q, k [B, H, N, D] (bf16 MFMA; see
    fib_dense_causal_lse)."""
    torch = _torch()
    _check_qkv(q, k)
    B, H, N, D = q.shape
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    need = int(lib().fib_dense_lse_workspace_size(B, H, N, D, _dtype_code(q)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib().fib_dense_causal_lse(_ptr(q), _ptr(k), _ptr(lse), B, H, N, D, _dtype_code(q),
                                    ctypes.c_float(float(theta)), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "fib_dense_causal_lse")
    return lse


@_on_stream
def dropped_mass(q, k, v, W: int, alpha, base: Sequence[int], theta: float = 10000.0, stream=None):
    """Per query, the dense causal softmax mass outside the integer-mode attended set:
    1 - exp(LSE_sparse - LSE_dense) [B, H, N] (three kernels: sparse forward, dense LSE, map)."""
    torch = _torch()
    _, lse_s = fwd(q, k, v, W, alpha, base, theta, INT, stream=stream)
    lse_d = dense_lse(q, k, theta, stream=stream)
    out = torch.empty_like(lse_s)
    st = lib().fib_sparse_attn_dropped_mass(_ptr(lse_s), _ptr(lse_d), _ptr(out), lse_s.numel(), _stream(stream))
    _check(st, "fib_sparse_attn_dropped_mass")
    return out


def bwd_workspace_size(B, H, N, D, dtype_code: int, mode: int, W: int = None, alpha_max=None, base=None) -> int:
    """Backward workspace bytes: for any base and alpha, or (W, alpha_max and base given) for
    calls with that W and base and alphas <= alpha_max."""
    if W is None:
        return int(lib().fib_sparse_attn_bwd_workspace_size(B, H, N, D, int(dtype_code), int(mode)))
    b, n = _base_array(base)
    return int(lib().fib_sparse_attn_bwd_workspace_size_for(B, H, N, D, int(dtype_code), int(mode), int(W),
                                                            ctypes.c_float(float(np.float32(alpha_max))), b, n))


@_on_stream
def bwd(q, k, v, o, lse, dout, W: int, alpha, base: Sequence[int], theta: float = 10000.0, mode: int = INT,
        dq=None, dk=None, dv=None, dalpha=None, workspace=None, want_dalpha: bool = True, stream=None):
    """Sparse attention backward; returns (dQ, dK, dV, dalpha tensor [1] or None)."""
    torch = _torch()
    _check_qkv(q, k, v, o, dout)
    B, H, N, D = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check_qkv(q, dq, dk, dv)
    if dalpha is None and want_dalpha:
        dalpha = torch.empty(1, dtype=torch.float32, device=q.device)
    need = bwd_workspace_size(B, H, N, D, _dtype_code(q), mode, W, alpha, base)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    b, n = _base_array(base)
    st = lib().fib_sparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dalpha), B, H, N, D, _dtype_code(q),
                                   int(W), ctypes.c_float(float(np.float32(alpha))), b, n,
                                   ctypes.c_float(float(theta)), int(mode), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "fib_sparse_attn_bwd")
    return dq, dk, dv, dalpha


NOALLOC_SCRATCH_BYTES = 64 << 20


@_on_stream
def bwd_noalloc(q, k, v, o, lse, dout, W: int, alpha, base: Sequence[int], theta: float = 10000.0, mode: int = INT,
                dq=None, dk=None, dv=None, dalpha=None, want_dalpha: bool = True, stream=None):
    """Backward through fib_sparse_attn_bwd_noalloc: no workspace (the library's fixed scratch,
    NOALLOC_SCRATCH_BYTES per GPU); returns (dQ, dK, dV, dalpha tensor [1] or None). Pass
    preallocated dq, dk, dv, dalpha to allocate nothing at all."""
    torch = _torch()
    _check_qkv(q, k, v, o, dout)
    B, H, N, D = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check_qkv(q, dq, dk, dv)
    if dalpha is None and want_dalpha:
        dalpha = torch.empty(1, dtype=torch.float32, device=q.device)
    b, n = _base_array(base)
    st = lib().fib_sparse_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                           _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dalpha), B, H, N, D, _dtype_code(q),
                                           int(W), ctypes.c_float(float(np.float32(alpha))), b, n,
                                           ctypes.c_float(float(theta)), int(mode), _stream(stream))
    _check(st, "fib_sparse_attn_bwd_noalloc")
    return dq, dk, dv, dalpha


@_on_stream
def index_set(N: int, W: int, alpha, base: Sequence[int], mode: int, device="cuda", stream=None):
    """Device export of the attended rows, int32 [N, W + n_entries] (-1 where absent)."""
    torch = _torch()
    dist, _, _ = offset_table(alpha, base, W, mode)
    cols = W + len(dist)
    out = torch.empty((N, cols), dtype=torch.int32, device=device)
    b, n = _base_array(base)
    st = lib().fib_sparse_attn_index_set(int(N), int(W), ctypes.c_float(float(np.float32(alpha))), b, n, int(mode),
                                         _ptr(out), cols, _stream(stream))
    _check(st, "fib_sparse_attn_index_set")
    return out
