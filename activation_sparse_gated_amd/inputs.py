"""Seeded synthetic inputs for the gate-first sparse FFN.

This module is shared by the HIP path's tests and bench and by the CPU oracle's
tests. It holds no FFN arithmetic: only random draws, the bf16 rounding of the
draws, and the constant that places a target fraction of gate pre-activations
below zero. Every array is generated from
``PCG64(SeedSequence([2026, cfg, layer, replica, stream]))``.

Recipe (the pages fix the FFN shapes but print no inputs, so these are our
choices, stated once here):

* Standard gating ("Model casting: compute the gate, then skip most of the
  FFN", section "What an FFN actually computes"): W1, W3 in R^{H x D} and W2 in
  R^{D x H}, every entry N(0, 1/D). W2 is stored transposed, W2T = W2^T with
  shape [H, D], so hidden unit i owns the contiguous row W2T[i].
* Tokens: x[0] = 1 and x[1:] ~ N(0, 1). Column 0 of W1 is set to
  c = -Phi^{-1}(s), so z_i = c + (a sum of D-1 terms of variance 1/D) and
  P(z_i > 0) = Phi(c) = 1 - s. A tiny workload fixes c = -1.2816 for s = 0.9.
* LoPA gating (same page, section "LoPA Gating: moving the ceiling"):
  V [r, D] ~ N(0, 1/D), U [H', r] ~ N(0, 1/r), W3 ~ N(0, 1/D),
  W2T [H', D] ~ N(0, 1/H'). The gate's bias rides on rank 0: V[0] = e_0 so
  (Vx)_0 = x_0 = 1, and U[:, 0] = c.
* Rounding: draw fp64, round to fp32, then round-to-nearest-even to bf16.
  Everything downstream consumes the bf16 values, so the quantisation is part
  of the input, not of the method.
"""
from __future__ import annotations

import numpy as np
from scipy.special import ndtri

SEED_BASE = 2026
# stream ids inside one (cfg, layer, replica) key
S_X, S_W1, S_W3, S_W2T, S_V, S_U = 0, 1, 2, 3, 4, 5


def rng(cfg: int, layer: int = 0, replica: int = 0, stream: int = 0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([SEED_BASE, cfg, layer, replica, stream])))


def to_bf16_bits(a) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (round to nearest, ties to even) as uint16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    out = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def gate_offset(sparsity: float) -> float:
    """c = -Phi^{-1}(s): with z ~ N(c, 1), P(z > 0) = 1 - s."""
    return float(-ndtri(sparsity))


def _finish(a64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return to_bf16_bits(a64)
    if dtype == "f32":
        return np.ascontiguousarray(a64.astype(np.float32))
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(shape, std: float, cfg: int, layer: int, replica: int, stream: int) -> np.ndarray:
    return rng(cfg, layer, replica, stream).standard_normal(size=shape, dtype=np.float64) * std


def tokens(D: int, n: int, cfg: int, layer: int = 0, replica: int = 0, dtype: str = "bf16",
           stream: int = S_X) -> np.ndarray:
    """n tokens [n, D]: x[:, 0] = 1, x[:, 1:] ~ N(0, 1)."""
    x = normal((n, D), 1.0, cfg, layer, replica, stream)
    x[:, 0] = 1.0
    return _finish(x, dtype)


def standard_weights(D: int, H: int, sparsity: float | None, cfg: int, layer: int = 0,
                     replica: int = 0, dtype: str = "bf16", offset: float | None = None) -> dict:
    """W1, W3, W2T, each [H, D], N(0, 1/D); W1[:, 0] = c sets the sparsity."""
    std = 1.0 / np.sqrt(D)
    W1 = normal((H, D), std, cfg, layer, replica, S_W1)
    c = offset if offset is not None else (gate_offset(sparsity) if sparsity is not None else None)
    if c is not None:
        W1[:, 0] = c
    W3 = normal((H, D), std, cfg, layer, replica, S_W3)
    W2T = normal((H, D), std, cfg, layer, replica, S_W2T)
    return {"W1": _finish(W1, dtype), "W3": _finish(W3, dtype), "W2T": _finish(W2T, dtype),
            "offset": c}


def quantize_rows_int8(w64: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric per-row int8 of a float matrix: scale_i = max_j |w_ij| / 127 (as fp32;
    1 for an all-zero row), q_ij = clip(rint(w_ij / scale_i), -127, 127). The weights
    the FFN then uses are q_ij * scale_i (the input recipe of the int8 workloads)."""
    amax = np.max(np.abs(w64), axis=1)
    scale = np.where(amax > 0, amax / 127.0, 1.0).astype(np.float32)
    q = np.clip(np.rint(w64 / scale.astype(np.float64)[:, None]), -127, 127).astype(np.int8)
    return np.ascontiguousarray(q), scale


def standard_weights_int8(D: int, H: int, sparsity: float | None, cfg: int, layer: int = 0,
                          replica: int = 0, offset: float | None = None) -> dict:
    """The fp64 draws of standard_weights (same streams, W1[:, 0] = c), quantized per
    row to int8: W1, W3, W2T int8 [H, D] and W1_scale, W3_scale, W2T_scale fp32 [H]."""
    std = 1.0 / np.sqrt(D)
    W1 = normal((H, D), std, cfg, layer, replica, S_W1)
    c = offset if offset is not None else (gate_offset(sparsity) if sparsity is not None else None)
    if c is not None:
        W1[:, 0] = c
    out = {"offset": c}
    for name, w in (("W1", W1), ("W3", normal((H, D), std, cfg, layer, replica, S_W3)),
                    ("W2T", normal((H, D), std, cfg, layer, replica, S_W2T))):
        out[name], out[name + "_scale"] = quantize_rows_int8(w)
    return out


S_ROUTE = 6


def moe_routing(T: int, E: int, K: int, cfg: int, layer: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Synthetic top-K routing: K distinct experts per token, uniform, and positive gate
    weights that sum to 1 per token (fp32). Returns route int32 [T, K], gate fp32 [T, K]."""
    g = rng(cfg, layer, 0, S_ROUTE)
    route = np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = g.random((T, K)) + 0.1
    gate = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return route, gate


def lopa_weights(D: int, Hp: int, r: int, sparsity: float | None, cfg: int, layer: int = 0,
                 replica: int = 0, dtype: str = "bf16", offset: float | None = None) -> dict:
    """V [r, D], U [Hp, r], W3 [Hp, D], W2T [Hp, D] with fan-in scaled variances."""
    V = normal((r, D), 1.0 / np.sqrt(D), cfg, layer, replica, S_V)
    U = normal((Hp, r), 1.0 / np.sqrt(r), cfg, layer, replica, S_U)
    c = offset if offset is not None else (gate_offset(sparsity) if sparsity is not None else None)
    if c is not None:
        V[0, :] = 0.0
        V[0, 0] = 1.0
        U[:, 0] = c
    W3 = normal((Hp, D), 1.0 / np.sqrt(D), cfg, layer, replica, S_W3)
    W2T = normal((Hp, D), 1.0 / np.sqrt(Hp), cfg, layer, replica, S_W2T)
    return {"V": _finish(V, dtype), "U": _finish(U, dtype), "W3": _finish(W3, dtype),
            "W2T": _finish(W2T, dtype), "offset": c}


INT4_GROUP = 128  # columns that share one int4 scale


def quantize_groups_int4(w64: np.ndarray, group: int = INT4_GROUP) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric int4 with one scale per `group` consecutive columns of a row:
    scale_ig = max |w| over the group / 7 (as fp32; 1 for an all-zero group),
    q = clip(rint(w / scale), -7, 7). Returns the codes packed two per byte (column 2j
    in the low nibble, 2j + 1 in the high nibble, two's complement), [H, D/2] uint8,
    and the scales [H, D/group] fp32. The weights the FFN then uses are q * scale."""
    H, D = w64.shape
    assert D % group == 0 and group % 2 == 0
    g = w64.reshape(H, D // group, group)
    amax = np.max(np.abs(g), axis=2)
    scale = np.where(amax > 0, amax / 7.0, 1.0).astype(np.float32)
    q = np.clip(np.rint(g / scale.astype(np.float64)[:, :, None]), -7, 7).astype(np.int8).reshape(H, D)
    packed = ((q[:, 0::2].astype(np.uint8) & 0xF) | ((q[:, 1::2].astype(np.uint8) & 0xF) << 4))
    return np.ascontiguousarray(packed.astype(np.uint8)), np.ascontiguousarray(scale)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """int4 codes [H, D] (int8) from the packed layout of quantize_groups_int4."""
    lo = (packed & 0xF).astype(np.int8)
    hi = (packed >> 4).astype(np.int8)
    lo = np.where(lo > 7, lo - 16, lo).astype(np.int8)
    hi = np.where(hi > 7, hi - 16, hi).astype(np.int8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def standard_weights_int4(D: int, H: int, sparsity: float | None, cfg: int, layer: int = 0,
                          replica: int = 0, offset: float | None = None) -> dict:
    """The fp64 draws of standard_weights (same streams, W1[:, 0] = c), quantized to
    int4 with one scale per 128 columns: W1, W3, W2T packed uint8 [H, D/2] and
    W1_scale, W3_scale, W2T_scale fp32 [H, D/128]."""
    std = 1.0 / np.sqrt(D)
    W1 = normal((H, D), std, cfg, layer, replica, S_W1)
    c = offset if offset is not None else (gate_offset(sparsity) if sparsity is not None else None)
    if c is not None:
        W1[:, 0] = c
    out = {"offset": c}
    for name, w in (("W1", W1), ("W3", normal((H, D), std, cfg, layer, replica, S_W3)),
                    ("W2T", normal((H, D), std, cfg, layer, replica, S_W2T))):
        out[name], out[name + "_scale"] = quantize_groups_int4(w)
    return out


def lopa_weights_int8(D: int, Hp: int, r: int, sparsity: float | None, cfg: int, layer: int = 0,
                      replica: int = 0, offset: float | None = None) -> dict:
    """The fp64 draws of lopa_weights (same streams, V[0] = e_0, U[:, 0] = c), quantized
    per row to int8: V, U, W3, W2T int8 and V_scale, U_scale, W3_scale, W2T_scale fp32."""
    V = normal((r, D), 1.0 / np.sqrt(D), cfg, layer, replica, S_V)
    U = normal((Hp, r), 1.0 / np.sqrt(r), cfg, layer, replica, S_U)
    c = offset if offset is not None else (gate_offset(sparsity) if sparsity is not None else None)
    if c is not None:
        V[0, :] = 0.0
        V[0, 0] = 1.0
        U[:, 0] = c
    out = {"offset": c}
    for name, w in (("V", V), ("U", U),
                    ("W3", normal((Hp, D), 1.0 / np.sqrt(D), cfg, layer, replica, S_W3)),
                    ("W2T", normal((Hp, D), 1.0 / np.sqrt(Hp), cfg, layer, replica, S_W2T))):
        out[name], out[name + "_scale"] = quantize_rows_int8(w)
    return out


def lopa_weights_int4(D: int, Hp: int, r: int, sparsity: float | None, cfg: int, layer: int = 0,
                      replica: int = 0, offset: float | None = None) -> dict:
    """The fp64 draws of lopa_weights (same streams, V[0] = e_0, U[:, 0] = c): V and U
    quantized per row to int8 (V, U int8 and V_scale, U_scale fp32), W3 and W2T to int4
    with one scale per 128 columns (packed uint8 [Hp, D/2], scales fp32 [Hp, D/128])."""
    V = normal((r, D), 1.0 / np.sqrt(D), cfg, layer, replica, S_V)
    U = normal((Hp, r), 1.0 / np.sqrt(r), cfg, layer, replica, S_U)
    c = offset if offset is not None else (gate_offset(sparsity) if sparsity is not None else None)
    if c is not None:
        V[0, :] = 0.0
        V[0, 0] = 1.0
        U[:, 0] = c
    out = {"offset": c}
    out["V"], out["V_scale"] = quantize_rows_int8(V)
    out["U"], out["U_scale"] = quantize_rows_int8(U)
    out["W3"], out["W3_scale"] = quantize_groups_int4(normal((Hp, D), 1.0 / np.sqrt(D), cfg, layer,
                                                             replica, S_W3))
    out["W2T"], out["W2T_scale"] = quantize_groups_int4(normal((Hp, D), 1.0 / np.sqrt(Hp), cfg,
                                                               layer, replica, S_W2T))
    return out


def small_integers(shape, lo: int, hi: int, cfg: int, layer: int = 0, replica: int = 0,
                   stream: int = 0, dtype: str = "bf16") -> np.ndarray:
    """Integers uniform in [lo, hi]; exact in bf16 and fp32 for |v| <= 256."""
    a = rng(cfg, layer, replica, stream).integers(lo, hi + 1, size=shape).astype(np.float64)
    return _finish(a, dtype)


def as_float(a: np.ndarray) -> np.ndarray:
    """View generated data as fp32 values (bf16 bits are widened exactly)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)
