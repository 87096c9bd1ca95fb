"""ctypes front end of the fp64 C oracle (sffn_oracle.c). Test infrastructure only.

Every function here evaluates the gated FFN of the page "Model casting: compute
the gate, then skip most of the FFN" (section "What an FFN actually computes")
one token at a time in fp64:

    z = W1 x              (standard)   or   z = U (V x)   (LoPA, section "LoPA Gating")
    h = A(z),  L = {i : z_i > 0}
    y = W2 (h (.) W3 x) = sum_{i in L} h_i (W3_i . x) W2T_i

Inputs are the generator's arrays: uint16 bf16 bit patterns, float32 or float64.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .buildlib import LIB, SRC, build as _build_lib

ACT_RELU, ACT_RSPLUS = 0, 1
_DT = {np.dtype(np.uint16): 0, np.dtype(np.float32): 1, np.dtype(np.float64): 2}
_lib = None


def build() -> str:
    global _lib
    _lib = None
    return _build_lib()


def _load(path: str | None = None):
    """Load the oracle library (the built one unless `path` names another build)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    if path is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            _build_lib()
        path = LIB
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.orc_activation.restype = ctypes.c_double
    lib.orc_activation.argtypes = [I, ctypes.c_double]
    lib.orc_num_threads.restype = I
    lib.orc_set_threads.argtypes = [I]
    lib.orc_ffn_standard.restype = I
    lib.orc_ffn_standard.argtypes = [I, I, I, I, P, P, P, P, I, P, P, P, P]
    lib.orc_ffn_lopa.restype = I
    lib.orc_ffn_lopa.argtypes = [I, I, I, I, I, P, P, P, P, P, I, P, P, P, P, P]
    if hasattr(lib, "orc_ffn_lopa_full"):  # older builds used by mutation tests may lack it
        lib.orc_ffn_lopa_full.restype = I
        lib.orc_ffn_lopa_full.argtypes = [I, I, I, I, I, ctypes.c_uint, P, P, P, P, P, I, P, P, P,
                                          P, P, P]
    _lib = lib
    return lib


class library:
    """Context manager that swaps in another build of the oracle (mutation tests)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.prev = _lib
        _load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.prev
        return False


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(*arrays) -> int:
    dts = {np.dtype(a.dtype) for a in arrays}
    if len(dts) != 1:
        raise TypeError(f"mixed input dtypes {dts}")
    dt = dts.pop()
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}")
    return _DT[dt]


def activation(act: int, z: float) -> float:
    """A(z): ReLU max(0, z), or R-S+ (z * sigmoid(z) for z >= 0, else 0)."""
    return _load().orc_activation(act, float(z))


def num_threads() -> int:
    return _load().orc_num_threads()


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def ffn_standard(x, W1, W3, W2T, act: int = ACT_RELU, dense: bool = False):
    """One token or a batch.

    x [D] or [T, D]; W1, W3, W2T [H, D]. Returns a dict with y [T, D] (fp64),
    z [T, H] (fp64 gate pre-activation), live (list of ascending int32 arrays)
    and k [T].
    """
    lib = _load()
    x2 = np.atleast_2d(np.ascontiguousarray(x))
    W1, W3, W2T = (np.ascontiguousarray(w) for w in (W1, W3, W2T))
    code = _dtype_code(x2, W1, W3, W2T)
    T, D = x2.shape
    H = W1.shape[0]
    if W1.shape != (H, D) or W3.shape != (H, D) or W2T.shape != (H, D):
        raise ValueError("weight shapes must all be [H, D]")
    y = np.zeros((T, D), np.float64)
    z = np.zeros((T, H), np.float64)
    idx = np.zeros(max(H, 1), np.int32)
    live, ks = [], np.zeros(T, np.int64)
    for t in range(T):
        k = lib.orc_ffn_standard(D, H, act, code, _ptr(x2[t]), _ptr(W1), _ptr(W3), _ptr(W2T),
                                 int(bool(dense)), _ptr(y[t]), _ptr(z[t]), None, _ptr(idx))
        if k < 0:
            raise RuntimeError(f"oracle failed ({k})")
        ks[t] = k
        live.append(idx[:k].copy())
    return {"y": y, "z": z, "live": live, "k": ks}


def ffn_lopa(x, V, U, W3, W2T, act: int = ACT_RELU, dense: bool = False):
    """LoPA gate z = U (V x); V [r, D], U [H, r], W3/W2T [H, D]. Adds t [T, r]."""
    lib = _load()
    x2 = np.atleast_2d(np.ascontiguousarray(x))
    V, U, W3, W2T = (np.ascontiguousarray(w) for w in (V, U, W3, W2T))
    code = _dtype_code(x2, V, U, W3, W2T)
    T, D = x2.shape
    r = V.shape[0]
    H = U.shape[0]
    if V.shape != (r, D) or U.shape != (H, r) or W3.shape != (H, D) or W2T.shape != (H, D):
        raise ValueError("LoPA shapes: V [r, D], U [H, r], W3/W2T [H, D]")
    y = np.zeros((T, D), np.float64)
    z = np.zeros((T, H), np.float64)
    tt = np.zeros((T, r), np.float64)
    idx = np.zeros(max(H, 1), np.int32)
    live, ks = [], np.zeros(T, np.int64)
    for t in range(T):
        k = lib.orc_ffn_lopa(D, H, r, act, code, _ptr(x2[t]), _ptr(V), _ptr(U), _ptr(W3),
                             _ptr(W2T), int(bool(dense)), _ptr(y[t]), _ptr(z[t]), _ptr(tt[t]),
                             None, _ptr(idx))
        if k < 0:
            raise RuntimeError(f"oracle failed ({k})")
        ks[t] = k
        live.append(idx[:k].copy())
    return {"y": y, "z": z, "t": tt, "live": live, "k": ks}


# flags of the full LoPA gate (page "Model casting: ...", section "LoPA Gating:
# moving the ceiling"; paper card Figure 6 and Table 4)
LOPA_G_TILED, LOPA_RMSNORM, LOPA_DOUBLE_ACT = 1, 2, 4
RMS_EPS = 1e-6  # not on the pages: the oracle's reading (unit gain as well)


def ffn_lopa_full(x, V, U, W3, W2T, flags: int, act: int = ACT_RELU, dense: bool = False):
    """Full LoPA gate z = G x + U RMSNorm(V x) with double activation, each part
    switched by `flags`. Returns y, z, t (after the norm), live, k, and k2 (units
    that enter the W2 pass)."""
    lib = _load()
    x2 = np.atleast_2d(np.ascontiguousarray(x))
    V, U, W3, W2T = (np.ascontiguousarray(w) for w in (V, U, W3, W2T))
    code = _dtype_code(x2, V, U, W3, W2T)
    T, D = x2.shape
    r = V.shape[0]
    H = U.shape[0]
    if V.shape != (r, D) or U.shape != (H, r) or W3.shape != (H, D) or W2T.shape != (H, D):
        raise ValueError("LoPA shapes: V [r, D], U [H, r], W3/W2T [H, D]")
    y = np.zeros((T, D), np.float64)
    z = np.zeros((T, H), np.float64)
    tt = np.zeros((T, r), np.float64)
    idx = np.zeros(max(H, 1), np.int32)
    k2 = np.zeros(1, np.int32)
    live, ks, k2s = [], np.zeros(T, np.int64), np.zeros(T, np.int64)
    for t in range(T):
        k = lib.orc_ffn_lopa_full(D, H, r, act, code, int(flags), _ptr(x2[t]), _ptr(V), _ptr(U),
                                  _ptr(W3), _ptr(W2T), int(bool(dense)), _ptr(y[t]), _ptr(z[t]),
                                  _ptr(tt[t]), None, _ptr(idx), _ptr(k2))
        if k < 0:
            raise RuntimeError(f"oracle failed ({k})")
        ks[t] = k
        k2s[t] = k2[0]
        live.append(idx[:k].copy())
    return {"y": y, "z": z, "t": tt, "live": live, "k": ks, "k2": k2s}


def dequantize_rows(q, scale):
    """Weights of a per-row int8 matrix as fp64: q_ij * scale_i (exact in fp64: an
    8-bit integer times an fp32 scale needs 32 significant bits)."""
    q = np.asarray(q)
    return q.astype(np.float64) * np.asarray(scale, np.float32).astype(np.float64)[:, None]


def ffn_standard_int8(x, w, act: int = ACT_RELU, dense: bool = False):
    """The standard oracle on the weights an int8 workload defines (q * scale per row);
    x is widened exactly to fp64. w: dict with W1/W3/W2T (int8) and *_scale (fp32)."""
    xf = np.atleast_2d(np.asarray(x))
    if xf.dtype == np.uint16:
        xf = (xf.astype(np.uint32) << 16).view(np.float32)
    xf = xf.astype(np.float64)
    return ffn_standard(xf, *(dequantize_rows(w[k], w[k + "_scale"]) for k in ("W1", "W3", "W2T")),
                        act=act, dense=dense)


def dequantize_groups_int4(packed, scale):
    """Weights of a group-scaled int4 matrix as fp64: code * scale of its group (exact
    in fp64). packed: [H, D/2] uint8, column 2j in the low nibble (two's complement);
    scale: [H, D/G] fp32."""
    packed = np.asarray(packed, np.uint8)
    H = packed.shape[0]
    D = packed.shape[1] * 2
    q = np.empty((H, D), np.int64)
    lo = (packed & 0xF).astype(np.int64)
    hi = (packed >> 4).astype(np.int64)
    q[:, 0::2] = np.where(lo >= 8, lo - 16, lo)
    q[:, 1::2] = np.where(hi >= 8, hi - 16, hi)
    scale = np.asarray(scale, np.float32).astype(np.float64)
    G = D // scale.shape[1]
    return q.astype(np.float64) * np.repeat(scale, G, axis=1)


def ffn_standard_int4(x, w, act: int = ACT_RELU, dense: bool = False):
    """The standard oracle on the weights a group-scaled int4 workload defines; x is
    widened exactly to fp64. w: dict with W1/W3/W2T (packed int4) and *_scale."""
    xf = np.atleast_2d(np.asarray(x))
    if xf.dtype == np.uint16:
        xf = (xf.astype(np.uint32) << 16).view(np.float32)
    xf = xf.astype(np.float64)
    return ffn_standard(xf, *(dequantize_groups_int4(w[k], w[k + "_scale"])
                              for k in ("W1", "W3", "W2T")), act=act, dense=dense)


def ffn_lopa_int8(x, w, act: int = ACT_RELU, flags: int = 0):
    """The LoPA oracle (flags as in ffn_lopa_full) on the weights an int8 LoPA workload
    defines: V, U, W3, W2T rows q * scale. x is widened exactly to fp64."""
    xf = np.atleast_2d(np.asarray(x))
    if xf.dtype == np.uint16:
        xf = (xf.astype(np.uint32) << 16).view(np.float32)
    xf = xf.astype(np.float64)
    V, U, W3, W2T = (dequantize_rows(w[k], w[k + "_scale"]) for k in ("V", "U", "W3", "W2T"))
    if flags:
        return ffn_lopa_full(xf, V, U, W3, W2T, flags, act=act)
    return ffn_lopa(xf, V, U, W3, W2T, act=act)


def ffn_lopa_int4(x, w, act: int = ACT_RELU, flags: int = 0):
    """The LoPA oracle (flags as in ffn_lopa_full) on the weights an int4 LoPA workload
    defines: V, U rows q * scale (int8), W3, W2T codes * their group's scale (int4). x is
    widened exactly to fp64."""
    xf = np.atleast_2d(np.asarray(x))
    if xf.dtype == np.uint16:
        xf = (xf.astype(np.uint32) << 16).view(np.float32)
    xf = xf.astype(np.float64)
    V, U = (dequantize_rows(w[k], w[k + "_scale"]) for k in ("V", "U"))
    W3, W2T = (dequantize_groups_int4(w[k], w[k + "_scale"]) for k in ("W3", "W2T"))
    if flags:
        return ffn_lopa_full(xf, V, U, W3, W2T, flags, act=act)
    return ffn_lopa(xf, V, U, W3, W2T, act=act)


def ffn_moe(x, experts, route, gate, act: int = ACT_RELU):
    """Top-K mixture of sparse FFN experts (page "Model casting: ...", section "Where it
    generalizes"): y_t = sum_k gate[t, k] * FFN_{route[t, k]}(x_t), k ascending, in fp64.
    experts: list of dicts with W1, W3, W2T."""
    x2 = np.atleast_2d(np.asarray(x))
    route = np.atleast_2d(np.asarray(route))
    gate = np.atleast_2d(np.asarray(gate, np.float64))
    T, D = x2.shape
    y = np.zeros((T, D), np.float64)
    for t in range(T):
        for k in range(route.shape[1]):
            w = experts[int(route[t, k])]
            o = ffn_standard(x2[t:t + 1], w["W1"], w["W3"], w["W2T"], act=act)
            y[t] += float(np.float32(gate[t, k])) * o["y"][0]
    return y
