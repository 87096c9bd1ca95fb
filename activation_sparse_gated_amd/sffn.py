"""Thin ctypes binding of libsffn.so (C ABI in include/sffn.h).

The functions keep the C names and only marshal arguments: torch tensors (or
raw integer addresses) become device pointers, and the current torch stream
becomes the `stream` argument unless one is given. Every step of the forward
pass runs in the library's HIP kernels; there is no fallback. If the library
has not been built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

SFFN_OK = 0
SFFN_INVALID_ARGUMENT = -1
SFFN_UNSUPPORTED = -2
SFFN_OUT_OF_MEMORY = -3
SFFN_HIP_ERROR = -4
SFFN_INTERNAL = -5

SFFN_ACT_RELU, SFFN_ACT_RSPLUS = 0, 1
SFFN_BF16, SFFN_F32, SFFN_I8, SFFN_I4 = 0, 1, 2, 3
SFFN_MODE_PER_TOKEN, SFFN_MODE_UNION = 0, 1
SFFN_FLAG_G_TILED, SFFN_FLAG_RMSNORM, SFFN_FLAG_DOUBLE_ACT = 1, 2, 4

EXPORTED = (
    "sffn_create", "sffn_destroy", "sffn_forward_dense", "sffn_forward_sparse",
    "sffn_forward_lopa", "sffn_last_error", "sffn_status_string", "sffn_abi_version",
    "sffn_timing_enable", "sffn_timing_read", "sffn_kernel_kinds", "sffn_kernel_name",
    "sffn_forward_sparse_i8", "sffn_forward_dense_i8", "sffn_forward_moe",
    "sffn_forward_lopa_i8", "sffn_forward_sparse_i4", "sffn_forward_dense_i4",
    "sffn_forward_lopa_i4", "sffn_forward_sparse_noalloc",
)

_lib = None


class SffnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


def library_path() -> str:
    return _build.LIB


def load() -> ctypes.CDLL:
    """Open libsffn.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P, I, U = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint
    PP = ctypes.POINTER(ctypes.c_void_p)
    lib.sffn_create.restype = I
    lib.sffn_create.argtypes = [PP, I, I, I, I, I, I, U]
    lib.sffn_destroy.restype = None
    lib.sffn_destroy.argtypes = [P]
    lib.sffn_forward_dense.restype = I
    lib.sffn_forward_dense.argtypes = [P, P, P, P, P, P, I, P]
    lib.sffn_forward_sparse.restype = I
    lib.sffn_forward_sparse.argtypes = [P, P, P, P, P, P, I, I, P, P, P]
    lib.sffn_forward_sparse_noalloc.restype = I
    lib.sffn_forward_sparse_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, P]
    lib.sffn_forward_lopa.restype = I
    lib.sffn_forward_lopa.argtypes = [P, P, P, P, P, P, P, I, I, P, P, P]
    lib.sffn_forward_sparse_i8.restype = I
    lib.sffn_forward_sparse_i8.argtypes = [P, P, P, P, P, P, P, P, P, I, I, P, P, P]
    lib.sffn_forward_sparse_i4.restype = I
    lib.sffn_forward_sparse_i4.argtypes = [P, P, P, P, P, P, P, P, P, I, I, P, P, P]
    lib.sffn_forward_dense_i4.restype = I
    lib.sffn_forward_dense_i4.argtypes = [P, P, P, P, P, P, P, P, P, I, P]
    lib.sffn_forward_lopa_i8.restype = I
    lib.sffn_forward_lopa_i8.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, P, P, P]
    lib.sffn_forward_lopa_i4.restype = I
    lib.sffn_forward_lopa_i4.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, P, P, P]
    lib.sffn_forward_dense_i8.restype = I
    lib.sffn_forward_dense_i8.argtypes = [P, P, P, P, P, P, P, P, P, I, P]
    lib.sffn_forward_moe.restype = I
    lib.sffn_forward_moe.argtypes = [P, P, I, PP, PP, PP, I, ctypes.POINTER(ctypes.c_int32),
                                     ctypes.POINTER(ctypes.c_float), P, I, I, P]
    lib.sffn_last_error.restype = ctypes.c_char_p
    lib.sffn_last_error.argtypes = [P]
    lib.sffn_status_string.restype = ctypes.c_char_p
    lib.sffn_status_string.argtypes = [I]
    lib.sffn_abi_version.restype = I
    lib.sffn_abi_version.argtypes = []
    lib.sffn_timing_enable.restype = I
    lib.sffn_timing_enable.argtypes = [P, I]
    lib.sffn_timing_read.restype = I
    lib.sffn_timing_read.argtypes = [P, I, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int64), I]
    lib.sffn_kernel_kinds.restype = I
    lib.sffn_kernel_kinds.argtypes = []
    lib.sffn_kernel_name.restype = ctypes.c_char_p
    lib.sffn_kernel_name.argtypes = [I]
    _lib = lib
    return lib


def _ptr(t):
    """Device address of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def status_string(status: int) -> str:
    return load().sffn_status_string(status).decode()


def sffn_last_error(handle=None) -> str:
    return load().sffn_last_error(handle).decode()


def sffn_abi_version() -> int:
    return load().sffn_abi_version()


def _check(status: int, handle) -> None:
    if status != SFFN_OK:
        raise SffnError(status, sffn_last_error(handle))


def sffn_create(D: int, H: int, r: int, max_tokens: int, act: int, dtype: int, flags: int = 0):
    """Returns the handle (an opaque address); raises SffnError on failure."""
    out = ctypes.c_void_p()
    st = load().sffn_create(ctypes.byref(out), D, H, r, max_tokens, act, dtype, flags)
    _check(st, None)
    return out.value


def sffn_create_status(D, H, r, max_tokens, act, dtype, flags=0):
    """Raw status form of sffn_create: (status, handle or None)."""
    out = ctypes.c_void_p()
    st = load().sffn_create(ctypes.byref(out), D, H, r, max_tokens, act, dtype, flags)
    return st, out.value


def sffn_destroy(handle) -> None:
    if handle:
        load().sffn_destroy(handle)


def sffn_forward_dense(handle, x, W1, W3, W2T, y, T: int, stream=None, check: bool = True) -> int:
    st = load().sffn_forward_dense(handle, _ptr(x), _ptr(W1), _ptr(W3), _ptr(W2T), _ptr(y), T,
                                   _stream(stream))
    if check:
        _check(st, handle)
    return st


def sffn_forward_sparse(handle, x, W1, W3, W2T, y, T: int, mode: int = SFFN_MODE_PER_TOKEN,
                        live_count=None, live_idx=None, stream=None, check: bool = True) -> int:
    st = load().sffn_forward_sparse(handle, _ptr(x), _ptr(W1), _ptr(W3), _ptr(W2T), _ptr(y), T,
                                    mode, _ptr(live_count), _ptr(live_idx), _stream(stream))
    if check:
        _check(st, handle)
    return st


def sffn_forward_sparse_noalloc(x, W1, W3, W2T, y, D: int, H: int, T: int, act: int,
                                stream=None, check: bool = True) -> int:
    st = load().sffn_forward_sparse_noalloc(_ptr(x), _ptr(W1), _ptr(W3), _ptr(W2T), _ptr(y), D, H,
                                            T, act, _stream(stream))
    if check:
        _check(st, None)
    return st


def sffn_forward_lopa(handle, x, V, U, W3, W2T, y, T: int, mode: int = SFFN_MODE_PER_TOKEN,
                      live_count=None, live_idx=None, stream=None, check: bool = True) -> int:
    st = load().sffn_forward_lopa(handle, _ptr(x), _ptr(V), _ptr(U), _ptr(W3), _ptr(W2T), _ptr(y),
                                  T, mode, _ptr(live_count), _ptr(live_idx), _stream(stream))
    if check:
        _check(st, handle)
    return st


def sffn_forward_sparse_i8(handle, x, W1, W1_scale, W3, W3_scale, W2T, W2T_scale, y, T: int,
                           mode: int = SFFN_MODE_PER_TOKEN, live_count=None, live_idx=None,
                           stream=None, check: bool = True) -> int:
    st = load().sffn_forward_sparse_i8(handle, _ptr(x), _ptr(W1), _ptr(W1_scale), _ptr(W3),
                                       _ptr(W3_scale), _ptr(W2T), _ptr(W2T_scale), _ptr(y), T,
                                       mode, _ptr(live_count), _ptr(live_idx), _stream(stream))
    if check:
        _check(st, handle)
    return st


def sffn_forward_sparse_i4(handle, x, W1, W1_scale, W3, W3_scale, W2T, W2T_scale, y, T: int,
                           mode: int = SFFN_MODE_PER_TOKEN, live_count=None, live_idx=None,
                           stream=None, check: bool = True) -> int:
    st = load().sffn_forward_sparse_i4(handle, _ptr(x), _ptr(W1), _ptr(W1_scale), _ptr(W3),
                                       _ptr(W3_scale), _ptr(W2T), _ptr(W2T_scale), _ptr(y), T,
                                       mode, _ptr(live_count), _ptr(live_idx), _stream(stream))
    if check:
        _check(st, handle)
    return st


def sffn_forward_dense_i4(handle, x, W1, W1_scale, W3, W3_scale, W2T, W2T_scale, y, T: int,
                          stream=None, check: bool = True) -> int:
    st = load().sffn_forward_dense_i4(handle, _ptr(x), _ptr(W1), _ptr(W1_scale), _ptr(W3),
                                      _ptr(W3_scale), _ptr(W2T), _ptr(W2T_scale), _ptr(y), T,
                                      _stream(stream))
    if check:
        _check(st, handle)
    return st


def sffn_forward_lopa_i8(handle, x, V, V_scale, U, U_scale, W3, W3_scale, W2T, W2T_scale, y,
                         T: int, mode: int = SFFN_MODE_PER_TOKEN, live_count=None, live_idx=None,
                         stream=None, check: bool = True) -> int:
    st = load().sffn_forward_lopa_i8(handle, _ptr(x), _ptr(V), _ptr(V_scale), _ptr(U),
                                     _ptr(U_scale), _ptr(W3), _ptr(W3_scale), _ptr(W2T),
                                     _ptr(W2T_scale), _ptr(y), T, mode, _ptr(live_count),
                                     _ptr(live_idx), _stream(stream))
    if check:
        _check(st, handle)
    return st


def sffn_forward_lopa_i4(handle, x, V, V_scale, U, U_scale, W3, W3_scale, W2T, W2T_scale, y,
                         T: int, mode: int = SFFN_MODE_PER_TOKEN, live_count=None, live_idx=None,
                         stream=None, check: bool = True) -> int:
    st = load().sffn_forward_lopa_i4(handle, _ptr(x), _ptr(V), _ptr(V_scale), _ptr(U),
                                     _ptr(U_scale), _ptr(W3), _ptr(W3_scale), _ptr(W2T),
                                     _ptr(W2T_scale), _ptr(y), T, mode, _ptr(live_count),
                                     _ptr(live_idx), _stream(stream))
    if check:
        _check(st, handle)
    return st


def sffn_forward_dense_i8(handle, x, W1, W1_scale, W3, W3_scale, W2T, W2T_scale, y, T: int,
                          stream=None, check: bool = True) -> int:
    st = load().sffn_forward_dense_i8(handle, _ptr(x), _ptr(W1), _ptr(W1_scale), _ptr(W3),
                                      _ptr(W3_scale), _ptr(W2T), _ptr(W2T_scale), _ptr(y), T,
                                      _stream(stream))
    if check:
        _check(st, handle)
    return st


def sffn_forward_moe(handle, x, W1s, W3s, W2Ts, route, gate, y, T: int, dense: bool = False,
                     stream=None, check: bool = True) -> int:
    """W1s/W3s/W2Ts: sequences of E device tensors (or addresses); route [T, K] int32 and
    gate [T, K] float32 are host arrays."""
    import numpy as np
    E = len(W1s)
    route = np.ascontiguousarray(route, dtype=np.int32)
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    K = route.shape[1] if route.ndim == 2 else 1
    arr = lambda ts: (ctypes.c_void_p * E)(*[_ptr(t) for t in ts])
    st = load().sffn_forward_moe(handle, _ptr(x), E, arr(W1s), arr(W3s), arr(W2Ts), K,
                                 route.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 gate.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _ptr(y), T,
                                 int(bool(dense)), _stream(stream))
    if check:
        _check(st, handle)
    return st


def sffn_timing_enable(handle, enable) -> None:
    """enable: False/0 off, True/1 every forward call, N > 1 every Nth call."""
    _check(load().sffn_timing_enable(handle, int(enable)), handle)


def sffn_timing_read(handle, kind: int, reset: bool = False):
    """(total milliseconds, launches) of kernel kind `kind` since the last reset."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(load().sffn_timing_read(handle, kind, ctypes.byref(ms), ctypes.byref(n), int(reset)),
           handle)
    return ms.value, n.value


def sffn_kernel_kinds() -> int:
    return load().sffn_kernel_kinds()


def sffn_kernel_name(kind: int) -> str:
    return load().sffn_kernel_name(kind).decode()


def kernel_kind(name: str) -> int:
    for k in range(sffn_kernel_kinds()):
        if sffn_kernel_name(k) == name:
            return k
    raise KeyError(name)


class Handle:
    """Owns one sffn handle; destroys it when closed or collected."""

    def __init__(self, D, H, r=0, max_tokens=1, act=SFFN_ACT_RELU, dtype=SFFN_BF16, flags=0):
        self.D, self.H, self.r, self.max_tokens = D, H, r, max_tokens
        self.act, self.dtype = act, dtype
        self.ptr = sffn_create(D, H, r, max_tokens, act, dtype, flags)

    def close(self):
        if self.ptr:
            sffn_destroy(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False
