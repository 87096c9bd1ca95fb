"""Pins for the fp64 CPU oracle (CPU only).

The oracle must be pinned to something other than itself. Each check below
ties it to a fact the pages or the mathematics fix:

* exact rational brute force on small integer inputs, written in the pages'
  column-vector convention (W2 is D x H, unit i owns column i), so a transposed
  operand, a dropped term, a wrong index or a wrong sign in the live test fails;
* the textbook ReLU and PyTorch's SiLU, which R-S+ must equal for z >= 0
  (page "Model casting: compute the gate, then skip most of the FFN", section
  "Model casting: make sparsity a target");
* the exactness of the skip (same page, section "What an FFN actually
  computes"): dense and sparse evaluation agree bitwise;
* closed-form special cases (every unit live, no unit live);
* LoPA's gate is W1 = UV when G is absent (section "LoPA Gating: moving the
  ceiling"), so materialising UV must reproduce the standard oracle;
* the input recipe's sparsity calibration, P(z > 0) = Phi(c);
* the full LoPA gate z = G x + U RMSNorm(V x) with double activation (same
  section; paper card Figure 6 (c) for the tiled identity G, Table 5 for the
  W2 skip): with G alone it is the standard FFN with W1 = T + UV materialised;
  exact rationals pin the double activation and the count of W2 rows it keeps;
  closed forms pin the RMSNorm (eps = 1e-6, unit gain, the oracle's reading).

``test_pins_catch_planted_mistakes`` plants plausible mistakes into copies of
the oracle's C source and checks that at least one pin fails for each.
"""
import math
import os
import shutil
import subprocess
import sys
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import reference as ref
from activation_sparse_gated_amd import inputs as gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# --------------------------------------------------------------------------- helpers
def frac_ffn(x, W1, W3, W2T, act_relu=True):
    """Exact rational FFN in the pages' convention: y = W2 (relu(W1 x) * (W3 x)).

    W2 is built as the D x H matrix whose column i is W2T[i]; products are
    written as explicit sums over plain Python lists of Fractions.
    """
    D = len(x)
    H = len(W1)
    W2 = [[Fraction(W2T[i][j]) for i in range(H)] for j in range(D)]   # D x H
    xs = [Fraction(v) for v in x]
    z = [sum(Fraction(W1[i][j]) * xs[j] for j in range(D)) for i in range(H)]
    g = [zi if zi > 0 else Fraction(0) for zi in z]
    u = [sum(Fraction(W3[i][j]) * xs[j] for j in range(D)) for i in range(H)]
    hid = [g[i] * u[i] for i in range(H)]
    y = [sum(W2[j][i] * hid[i] for i in range(H)) for j in range(D)]
    live = [i for i in range(H) if z[i] > 0]
    return y, z, live


def int_case(D, H, T, seed, lo=-3, hi=3, dtype="bf16"):
    x = gen.small_integers((T, D), lo, hi, cfg=900 + seed, stream=0, dtype=dtype)
    W1 = gen.small_integers((H, D), lo, hi, cfg=900 + seed, stream=1, dtype=dtype)
    W3 = gen.small_integers((H, D), lo, hi, cfg=900 + seed, stream=2, dtype=dtype)
    W2T = gen.small_integers((H, D), lo, hi, cfg=900 + seed, stream=3, dtype=dtype)
    return x, W1, W3, W2T


def check_bruteforce():
    """Oracle == exact rationals on integer inputs, for bf16, f32 and f64 storage."""
    for (D, H, T, seed) in [(8, 12, 3, 1), (16, 40, 2, 2), (5, 3, 2, 3)]:
        for dtype in ("bf16", "f32"):
            x, W1, W3, W2T = int_case(D, H, T, seed, dtype=dtype)
            xf, W1f, W3f, W2Tf = (gen.as_float(a).astype(np.float64) for a in (x, W1, W3, W2T))
            for dense in (False, True):
                got = ref.ffn_standard(x, W1, W3, W2T, act=ref.ACT_RELU, dense=dense)
                got64 = ref.ffn_standard(xf, W1f, W3f, W2Tf, act=ref.ACT_RELU, dense=dense)
                for t in range(T):
                    xi = [int(v) for v in xf[t]]
                    y, z, live = frac_ffn(xi, W1f.astype(int).tolist(), W3f.astype(int).tolist(),
                                          W2Tf.astype(int).tolist())
                    for res in (got, got64):
                        assert [Fraction(v) for v in res["y"][t]] == y
                        assert [Fraction(v) for v in res["z"][t]] == z
                        assert res["live"][t].tolist() == live
                        assert res["k"][t] == len(live)


def check_numpy_float():
    """Random real inputs: oracle vs numpy's fp64 matrix products, both activations."""
    rng = np.random.default_rng(7)
    for (D, H) in [(8, 16), (24, 9)]:
        x = rng.standard_normal((2, D))
        W1 = rng.standard_normal((H, D))
        W3 = rng.standard_normal((H, D))
        W2 = rng.standard_normal((D, H))          # the pages' D x H down projection
        W2T = np.ascontiguousarray(W2.T)
        for act in (ref.ACT_RELU, ref.ACT_RSPLUS):
            got = ref.ffn_standard(x, W1, W3, W2T, act=act)
            for t in range(2):
                z = W1 @ x[t]
                g = torch.relu(torch.from_numpy(z)).numpy() if act == ref.ACT_RELU else \
                    np.where(z >= 0, torch.nn.functional.silu(torch.from_numpy(z)).numpy(), 0.0)
                y = W2 @ (g * (W3 @ x[t]))
                np.testing.assert_allclose(got["y"][t], y, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(got["z"][t], z, rtol=1e-13, atol=1e-13)
                assert got["live"][t].tolist() == np.flatnonzero(z > 0).tolist()


def check_rsplus():
    zs = np.concatenate([np.linspace(-40, 40, 801), [0.0, -0.0, 1e-300, -1e-300, 700.0, -700.0]])
    silu = torch.nn.functional.silu(torch.from_numpy(zs.astype(np.float64))).numpy()
    for z, s in zip(zs, silu):
        v = ref.activation(ref.ACT_RSPLUS, z)
        if z >= 0:
            assert abs(v - s) <= 1e-15 * max(1.0, abs(s)), (z, v, s)
        else:
            assert v == 0.0
        assert v >= 0.0
        assert ref.activation(ref.ACT_RELU, z) == max(0.0, z)
    assert ref.activation(ref.ACT_RSPLUS, 0.0) == 0.0
    assert ref.activation(ref.ACT_RSPLUS, 1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), abs=1e-16)


def check_lopa_is_standard_with_uv():
    # integers: exact
    D, H, r = 12, 20, 4
    x = gen.small_integers((2, D), -2, 2, cfg=950, stream=0, dtype="f32").astype(np.float64)
    V = gen.small_integers((r, D), -2, 2, cfg=950, stream=4, dtype="f32").astype(np.float64)
    U = gen.small_integers((H, r), -2, 2, cfg=950, stream=5, dtype="f32").astype(np.float64)
    W3 = gen.small_integers((H, D), -2, 2, cfg=950, stream=2, dtype="f32").astype(np.float64)
    W2T = gen.small_integers((H, D), -2, 2, cfg=950, stream=3, dtype="f32").astype(np.float64)
    W1 = U @ V
    a = ref.ffn_lopa(x, V, U, W3, W2T)
    b = ref.ffn_standard(x, W1, W3, W2T)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["z"], b["z"])
    assert all(np.array_equal(p, q) for p, q in zip(a["live"], b["live"]))
    np.testing.assert_array_equal(a["t"], x @ V.T)
    # real values, both activations
    rng = np.random.default_rng(11)
    D, H, r = 32, 48, 8
    x = rng.standard_normal((2, D))
    V, U = rng.standard_normal((r, D)), rng.standard_normal((H, r))
    W3, W2T = rng.standard_normal((H, D)), rng.standard_normal((H, D))
    for act in (ref.ACT_RELU, ref.ACT_RSPLUS):
        a = ref.ffn_lopa(x, V, U, W3, W2T, act=act)
        b = ref.ffn_standard(x, U @ V, W3, W2T, act=act)
        np.testing.assert_allclose(a["z"], b["z"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(a["y"], b["y"], rtol=1e-11, atol=1e-11)


def check_dense_equals_sparse():
    D, H = 256, 704
    x = gen.tokens(D, 4, cfg=1, dtype="f32")
    w = gen.standard_weights(D, H, None, cfg=1, dtype="f32", offset=-1.2816)
    for act in (ref.ACT_RELU, ref.ACT_RSPLUS):
        s = ref.ffn_standard(x, w["W1"], w["W3"], w["W2T"], act=act, dense=False)
        d = ref.ffn_standard(x, w["W1"], w["W3"], w["W2T"], act=act, dense=True)
        assert np.array_equal(s["y"].view(np.uint64), d["y"].view(np.uint64))
        assert 0 < s["k"].min() and s["k"].max() < H


def check_all_and_none_live():
    D, H = 64, 96
    x = gen.tokens(D, 3, cfg=77, dtype="bf16")
    for act in (ref.ACT_RELU, ref.ACT_RSPLUS):
        w = gen.standard_weights(D, H, None, cfg=77, dtype="bf16", offset=50.0)
        s = ref.ffn_standard(x, w["W1"], w["W3"], w["W2T"], act=act)
        d = ref.ffn_standard(x, w["W1"], w["W3"], w["W2T"], act=act, dense=True)
        assert (s["k"] == H).all()
        assert np.array_equal(s["y"], d["y"])
        # with every unit live the FFN is the plain gated product
        xf = gen.as_float(x).astype(np.float64)
        W1, W3, W2T = (gen.as_float(w[k]).astype(np.float64) for k in ("W1", "W3", "W2T"))
        for t in range(3):
            z = W1 @ xf[t]
            g = z if act == ref.ACT_RELU else z / (1 + np.exp(-z))
            np.testing.assert_allclose(s["y"][t], W2T.T @ (g * (W3 @ xf[t])), rtol=1e-12)
        w = gen.standard_weights(D, H, None, cfg=77, dtype="bf16", offset=-50.0)
        s = ref.ffn_standard(x, w["W1"], w["W3"], w["W2T"], act=act)
        assert (s["k"] == 0).all()
        assert np.all(s["y"] == 0.0) and not np.any(np.signbit(s["y"]))


def tiled_identity(H, D):
    """The paper card's Figure 6 (c): T[i][i mod D] = 1, every other entry 0."""
    Tm = np.zeros((H, D))
    for i in range(H):
        Tm[i, i % D] = 1.0
    return Tm


def check_lopa_full_g_is_materialised_gate():
    """G alone: the full LoPA oracle equals the standard oracle with W1 = T + UV."""
    rng = np.random.default_rng(21)
    for (D, H, r) in [(16, 40, 4), (24, 24, 8), (8, 19, 8)]:
        x = rng.standard_normal((3, D))
        V, U = rng.standard_normal((r, D)) * 0.3, rng.standard_normal((H, r)) * 0.3
        W3, W2T = rng.standard_normal((H, D)), rng.standard_normal((H, D))
        for act in (ref.ACT_RELU, ref.ACT_RSPLUS):
            a = ref.ffn_lopa_full(x, V, U, W3, W2T, ref.LOPA_G_TILED, act=act)
            b = ref.ffn_standard(x, tiled_identity(H, D) + U @ V, W3, W2T, act=act)
            np.testing.assert_allclose(a["z"], b["z"], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(a["y"], b["y"], rtol=1e-11, atol=1e-11)
            assert all(np.array_equal(p, q) for p, q in zip(a["live"], b["live"]))
    # integers: exact, G included
    D, H, r = 6, 14, 3
    x = gen.small_integers((2, D), -2, 2, cfg=951, stream=0, dtype="f32").astype(np.float64)
    V = gen.small_integers((r, D), -2, 2, cfg=951, stream=4, dtype="f32").astype(np.float64)
    U = gen.small_integers((H, r), -2, 2, cfg=951, stream=5, dtype="f32").astype(np.float64)
    W3 = gen.small_integers((H, D), -2, 2, cfg=951, stream=2, dtype="f32").astype(np.float64)
    W2T = gen.small_integers((H, D), -2, 2, cfg=951, stream=3, dtype="f32").astype(np.float64)
    a = ref.ffn_lopa_full(x, V, U, W3, W2T, ref.LOPA_G_TILED)
    b = ref.ffn_standard(x, tiled_identity(H, D) + U @ V, W3, W2T)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["z"], b["z"])


def frac_lopa_double(x, V, U, W3, W2T, g_tiled):
    """Exact rationals: z = [G x] + U (V x), a_i = relu(z_i) * relu(u_i), y = W2 a.
    Returns y, the live set and the number of live units with a_i != 0."""
    D, H, r = len(x), len(U), len(V)
    xs = [Fraction(v) for v in x]
    t = [sum(Fraction(V[m][j]) * xs[j] for j in range(D)) for m in range(r)]
    z = [(xs[i % D] if g_tiled else Fraction(0)) + sum(Fraction(U[i][m]) * t[m] for m in range(r))
         for i in range(H)]
    u = [sum(Fraction(W3[i][j]) * xs[j] for j in range(D)) for i in range(H)]
    a = [(z[i] if z[i] > 0 else 0) * (u[i] if u[i] > 0 else 0) for i in range(H)]
    W2 = [[Fraction(W2T[i][j]) for i in range(H)] for j in range(D)]
    y = [sum(W2[j][i] * a[i] for i in range(H)) for j in range(D)]
    live = [i for i in range(H) if z[i] > 0]
    return y, live, sum(1 for i in live if a[i] != 0)


def check_lopa_full_double_act_exact():
    """Double activation (ReLU) on integer inputs: y, L and the kept W2 rows, exactly."""
    for (D, H, r, seed) in [(6, 14, 3, 1), (10, 20, 5, 2)]:
        x = gen.small_integers((3, D), -2, 2, cfg=960 + seed, stream=0, dtype="bf16")
        V = gen.small_integers((r, D), -2, 2, cfg=960 + seed, stream=4, dtype="bf16")
        U = gen.small_integers((H, r), -2, 2, cfg=960 + seed, stream=5, dtype="bf16")
        W3 = gen.small_integers((H, D), -2, 2, cfg=960 + seed, stream=2, dtype="bf16")
        W2T = gen.small_integers((H, D), -2, 2, cfg=960 + seed, stream=3, dtype="bf16")
        f = [gen.as_float(a).astype(np.float64) for a in (x, V, U, W3, W2T)]
        for g in (False, True):
            flags = ref.LOPA_DOUBLE_ACT | (ref.LOPA_G_TILED if g else 0)
            for dense in (False, True):
                got = ref.ffn_lopa_full(x, V, U, W3, W2T, flags, dense=dense)
                for t in range(3):
                    y, live, k2 = frac_lopa_double([int(v) for v in f[0][t]],
                                                   *(m.astype(int).tolist() for m in f[1:]), g)
                    assert [Fraction(v) for v in got["y"][t]] == y
                    assert got["live"][t].tolist() == live
                    if not dense:
                        assert got["k2"][t] == k2 <= len(live)


def check_lopa_full_double_act_reduces_to_single():
    """When every u_i = W3_i . x > 0, A(u_i) = u_i for ReLU: double == single activation."""
    rng = np.random.default_rng(23)
    D, H, r = 20, 30, 5
    x = rng.standard_normal((2, D))
    V, U = rng.standard_normal((r, D)), rng.standard_normal((H, r))
    W2T = rng.standard_normal((H, D))
    for t in range(2):
        W3 = np.abs(rng.standard_normal((H, D))) * np.sign(x[t])[None, :]   # u_i > 0 for token t
        a = ref.ffn_lopa_full(x[t:t + 1], V, U, W3, W2T, ref.LOPA_DOUBLE_ACT)
        b = ref.ffn_lopa_full(x[t:t + 1], V, U, W3, W2T, 0)
        assert np.array_equal(a["y"], b["y"]) and a["k2"][0] == a["k"][0]


def check_lopa_full_rmsnorm():
    """RMSNorm(t) = t / sqrt(mean t^2 + eps): a constant t gives c / sqrt(c^2 + eps) in
    every entry; for any t, mean(RMSNorm(t)^2) = ms / (ms + eps) with ms = mean t^2."""
    eps = ref.RMS_EPS
    D, H, r = 16, 24, 8
    rng = np.random.default_rng(29)
    U = rng.standard_normal((H, r))
    W3, W2T = rng.standard_normal((H, D)), rng.standard_normal((H, D))
    x = rng.standard_normal((1, D))
    x[0, 0] = 1.0
    for c in (3.0, 1e-3, -0.25):
        V = np.zeros((r, D))
        V[:, 0] = c                                   # t_m = c * x_0 = c for every m
        o = ref.ffn_lopa_full(x, V, U, W3, W2T, ref.LOPA_RMSNORM)
        tn = c / math.sqrt(c * c + eps)
        np.testing.assert_allclose(o["t"][0], np.full(r, tn), rtol=1e-14)
        np.testing.assert_allclose(o["z"][0], U.sum(axis=1) * tn, rtol=1e-12, atol=1e-14)
    V = rng.standard_normal((r, D)) * 0.01
    o = ref.ffn_lopa_full(x, V, U, W3, W2T, ref.LOPA_RMSNORM)
    raw = ref.ffn_lopa_full(x, V, U, W3, W2T, 0)["t"][0]
    ms = float(np.mean(raw ** 2))
    assert float(np.mean(o["t"][0] ** 2)) == pytest.approx(ms / (ms + eps), rel=1e-12)
    np.testing.assert_allclose(o["t"][0], raw / math.sqrt(ms + eps), rtol=1e-12)


# --------------------------------------------------------------------------- tests
def test_bruteforce_exact():
    check_bruteforce()


def test_numpy_float_products():
    check_numpy_float()


def test_rsplus_and_relu():
    check_rsplus()


def test_lopa_reduces_to_standard():
    check_lopa_is_standard_with_uv()


def test_lopa_full_g_is_materialised_gate():
    check_lopa_full_g_is_materialised_gate()


def test_lopa_full_double_act_exact():
    check_lopa_full_double_act_exact()


def test_lopa_full_double_act_reduces_to_single():
    check_lopa_full_double_act_reduces_to_single()


def test_lopa_full_rmsnorm():
    check_lopa_full_rmsnorm()


def test_int8_weights_are_rows_times_scales():
    """An int8 workload's weights are q_ij * scale_i: exact in fp64, within half a step
    of the fp64 draw, and the oracle on them equals exact rationals for integer q."""
    w = gen.standard_weights_int8(64, 96, 0.9, cfg=70)
    w64 = gen.normal((96, 64), 1.0 / 8.0, 70, 0, 0, gen.S_W3)
    deq = ref.dequantize_rows(w["W3"], w["W3_scale"])
    step = w["W3_scale"].astype(np.float64)[:, None]
    assert np.all(np.abs(deq - w64) <= 0.5 * step * (1 + 1e-12))
    assert np.abs(w["W3"]).max() == 127
    for k in ("W1", "W3", "W2T"):
        assert w[k].dtype == np.int8 and w[k + "_scale"].dtype == np.float32
    # power-of-two scales: exact, and the FFN on them is exact rationals
    D, H = 8, 12
    q = {k: gen.small_integers((H, D), -3, 3, cfg=71, stream=s, dtype="f32").astype(np.int8)
         for k, s in (("W1", 1), ("W3", 2), ("W2T", 3))}
    x = gen.small_integers((2, D), -2, 2, cfg=71, stream=0, dtype="bf16")
    sc = {k: np.full(H, 2.0 ** -e, np.float32) for k, e in (("W1", 1), ("W3", 2), ("W2T", 3))}
    wi = {**q, **{k + "_scale": v for k, v in sc.items()}}
    got = ref.ffn_standard_int8(x, wi)
    xf = gen.as_float(x).astype(np.float64)
    for t in range(2):
        y, z, live = frac_ffn([Fraction(v) for v in xf[t]],
                              [[Fraction(int(v)) * Fraction(1, 2) for v in row] for row in q["W1"]],
                              [[Fraction(int(v)) * Fraction(1, 4) for v in row] for row in q["W3"]],
                              [[Fraction(int(v)) * Fraction(1, 8) for v in row] for row in q["W2T"]])
        assert [Fraction(v) for v in got["y"][t]] == y
        assert got["live"][t].tolist() == live


def test_lopa_int8_weights_and_exact_oracle():
    """An int8 LoPA workload's V, U, W3, W2T are rows q * scale (within half a step of the
    fp64 draws, V[0] = e_0 exactly representable), and the int8 LoPA oracle equals exact
    rationals on small integer codes with power-of-two scales: the plain gate U (V x), and
    G x + U (V x) with double activation."""
    D, Hp, r = 64, 80, 16
    w = gen.lopa_weights_int8(D, Hp, r, 0.9, cfg=72)
    U64 = gen.normal((Hp, r), 1.0 / np.sqrt(r), 72, 0, 0, gen.S_U)
    U64[:, 0] = w["offset"]
    deq = ref.dequantize_rows(w["U"], w["U_scale"])
    assert np.all(np.abs(deq - U64) <= 0.5 * w["U_scale"].astype(np.float64)[:, None] * (1 + 1e-12))
    assert w["V"][0, 0] == 127 and not w["V"][0, 1:].any()
    for k in ("V", "U", "W3", "W2T"):
        assert w[k].dtype == np.int8 and w[k + "_scale"].dtype == np.float32
    D, H, r = 6, 10, 4
    shapes = {"V": (r, D), "U": (H, r), "W3": (H, D), "W2T": (H, D)}
    q = {k: gen.small_integers(sh, -3, 3, cfg=73, stream=i + 1, dtype="f32").astype(np.int8)
         for i, (k, sh) in enumerate(shapes.items())}
    sc = {"V": 0.5, "U": 0.25, "W3": 0.5, "W2T": 0.125}
    wi = {**q, **{k + "_scale": np.full(shapes[k][0], v, np.float32) for k, v in sc.items()}}
    x = gen.small_integers((2, D), -2, 2, cfg=73, stream=0, dtype="bf16")
    xf = gen.as_float(x).astype(np.float64)
    mats = {k: [[Fraction(int(v)) * Fraction(sc[k]) for v in row] for row in q[k]] for k in q}
    plain = ref.ffn_lopa_int8(x, wi)
    full = ref.ffn_lopa_int8(x, wi, flags=ref.LOPA_G_TILED | ref.LOPA_DOUBLE_ACT)
    for t in range(2):
        xs = [Fraction(v) for v in xf[t]]
        tt = [sum(mats["V"][m][j] * xs[j] for j in range(D)) for m in range(r)]
        z = [sum(mats["U"][i][m] * tt[m] for m in range(r)) for i in range(H)]
        u = [sum(mats["W3"][i][j] * xs[j] for j in range(D)) for i in range(H)]
        a = [(z[i] if z[i] > 0 else 0) * u[i] for i in range(H)]
        y = [sum(mats["W2T"][i][j] * a[i] for i in range(H)) for j in range(D)]
        assert [Fraction(v) for v in plain["y"][t]] == y
        assert plain["live"][t].tolist() == [i for i in range(H) if z[i] > 0]
        yd, live_d, k2 = frac_lopa_double(xs, mats["V"], mats["U"], mats["W3"], mats["W2T"], True)
        assert [Fraction(v) for v in full["y"][t]] == yd
        assert full["live"][t].tolist() == live_d and full["k2"][t] == k2


def test_int4_packing_scales_and_exact_oracle():
    """A group-scaled int4 workload: the packed nibbles decode (brute force, per element)
    to the codes both unpackers return; every weight is within half a step of its fp64
    draw; and the int4 oracle equals exact rationals for integer codes with a different
    power-of-two scale in each 128-column group."""
    D, H = 256, 24
    w = gen.standard_weights_int4(D, H, 0.9, cfg=74)
    w64 = gen.normal((H, D), 1.0 / 16.0, 74, 0, 0, gen.S_W3)
    codes = gen.unpack_int4(w["W3"])
    for i in range(3):
        for j in range(D):
            byte = int(w["W3"][i, j // 2])
            nib = (byte >> 4) if j % 2 else (byte & 0xF)
            assert codes[i, j] == (nib - 16 if nib >= 8 else nib)
    assert np.abs(codes).max() == 7 and codes.min() >= -7
    deq = ref.dequantize_groups_int4(w["W3"], w["W3_scale"])
    step = np.repeat(w["W3_scale"].astype(np.float64), 128, axis=1)
    assert np.all(np.abs(deq - w64) <= 0.5 * step * (1 + 1e-12))
    assert np.array_equal(deq, codes.astype(np.float64) * step)
    # integer codes, a power-of-two scale per group: exact rationals
    D, H, T = 256, 6, 2
    rngq = np.random.default_rng(75)
    q = {k: rngq.integers(-8, 8, size=(H, D)).astype(np.int8) for k in ("W1", "W3", "W2T")}
    packed = {k: ((v[:, 0::2].astype(np.uint8) & 0xF) | ((v[:, 1::2].astype(np.uint8) & 0xF) << 4))
              for k, v in q.items()}
    sc = {k: (2.0 ** -rngq.integers(0, 4, size=(H, D // 128))).astype(np.float32) for k in q}
    wi = {**packed, **{k + "_scale": v for k, v in sc.items()}}
    x = gen.small_integers((T, D), -1, 1, cfg=75, stream=0, dtype="bf16")
    got = ref.ffn_standard_int4(x, wi)
    xf = gen.as_float(x).astype(np.float64)
    mats = {k: [[Fraction(int(q[k][i, j])) * Fraction(float(sc[k][i, j // 128])) for j in range(D)]
                for i in range(H)] for k in q}
    for t in range(T):
        y, z, live = frac_ffn([Fraction(v) for v in xf[t]], mats["W1"], mats["W3"], mats["W2T"])
        assert [Fraction(v) for v in got["y"][t]] == y
        assert got["live"][t].tolist() == live


def test_lopa_int4_weights_and_exact_oracle():
    """An int4 LoPA workload: V and U are int8 rows q * scale (V[0] = e_0 exactly), W3 and
    W2T int4 codes times their 128-column group's scale, each within half a step of the
    fp64 draws; and the int4 LoPA oracle equals exact rationals on integer codes with
    power-of-two scales (a different one per group of W3 and W2T): the plain gate
    U (V x), and G x + U (V x) with double activation."""
    D, Hp, r = 256, 40, 16
    w = gen.lopa_weights_int4(D, Hp, r, 0.9, cfg=76)
    assert w["V"][0, 0] == 127 and not w["V"][0, 1:].any()
    for k in ("V", "U"):
        assert w[k].dtype == np.int8 and w[k + "_scale"].shape == (w[k].shape[0],)
    for k in ("W3", "W2T"):
        assert w[k].dtype == np.uint8 and w[k].shape == (Hp, D // 2)
        assert w[k + "_scale"].shape == (Hp, D // 128)
    W2T64 = gen.normal((Hp, D), 1.0 / np.sqrt(Hp), 76, 0, 0, gen.S_W2T)
    deq = ref.dequantize_groups_int4(w["W2T"], w["W2T_scale"])
    step = np.repeat(w["W2T_scale"].astype(np.float64), 128, axis=1)
    assert np.all(np.abs(deq - W2T64) <= 0.5 * step * (1 + 1e-12))
    D, H, r, T = 256, 6, 4, 2
    rngq = np.random.default_rng(77)
    qV = rngq.integers(-3, 4, size=(r, D)).astype(np.int8)
    qU = rngq.integers(-3, 4, size=(H, r)).astype(np.int8)
    q4 = {k: rngq.integers(-8, 8, size=(H, D)).astype(np.int8) for k in ("W3", "W2T")}
    sc4 = {k: (2.0 ** -rngq.integers(0, 4, size=(H, D // 128))).astype(np.float32) for k in q4}
    wi = {"V": qV, "V_scale": np.full(r, 0.5, np.float32), "U": qU,
          "U_scale": np.full(H, 0.25, np.float32)}
    for k, v in q4.items():
        wi[k] = ((v[:, 0::2].astype(np.uint8) & 0xF) | ((v[:, 1::2].astype(np.uint8) & 0xF) << 4))
        wi[k + "_scale"] = sc4[k]
    x = gen.small_integers((T, D), -1, 1, cfg=77, stream=0, dtype="bf16")
    xf = gen.as_float(x).astype(np.float64)
    mats = {"V": [[Fraction(int(v)) * Fraction(1, 2) for v in row] for row in qV],
            "U": [[Fraction(int(v)) * Fraction(1, 4) for v in row] for row in qU]}
    for k in q4:
        mats[k] = [[Fraction(int(q4[k][i, j])) * Fraction(float(sc4[k][i, j // 128])) for j in range(D)]
                   for i in range(H)]
    plain = ref.ffn_lopa_int4(x, wi)
    full = ref.ffn_lopa_int4(x, wi, flags=ref.LOPA_G_TILED | ref.LOPA_DOUBLE_ACT)
    for t in range(T):
        xs = [Fraction(v) for v in xf[t]]
        tt = [sum(mats["V"][m][j] * xs[j] for j in range(D)) for m in range(r)]
        z = [sum(mats["U"][i][m] * tt[m] for m in range(r)) for i in range(H)]
        u = [sum(mats["W3"][i][j] * xs[j] for j in range(D)) for i in range(H)]
        a = [(z[i] if z[i] > 0 else 0) * u[i] for i in range(H)]
        y = [sum(mats["W2T"][i][j] * a[i] for i in range(H)) for j in range(D)]
        assert [Fraction(v) for v in plain["y"][t]] == y
        assert plain["live"][t].tolist() == [i for i in range(H) if z[i] > 0]
        yd, live_d, k2 = frac_lopa_double(xs, mats["V"], mats["U"], mats["W3"], mats["W2T"], True)
        assert [Fraction(v) for v in full["y"][t]] == yd
        assert full["live"][t].tolist() == live_d and full["k2"][t] == k2


def test_moe_exact_on_integers():
    """Top-K mixture (page "Model casting: ...", section "Where it generalizes"): y_t is the
    gate-weighted sum of the routed experts' FFN outputs, checked with exact rationals on
    small integers and dyadic gates, K = 1 and 2, with an expert no token uses."""
    D, H, E, T = 6, 10, 4, 5
    experts = []
    for e in range(E):
        _, W1, W3, W2T = int_case(D, H, 1, 40 + e)
        experts.append({"W1": W1, "W3": W3, "W2T": W2T})
    x = int_case(D, H, T, 50)[0]
    xf = gen.as_float(x).astype(np.float64)
    route2 = np.array([[0, 2], [2, 0], [1, 2], [0, 1], [2, 1]], np.int32)   # expert 3 unused
    gate2 = np.array([[0.75, 0.25], [0.5, 0.5], [1.0, 0.125], [0.375, 0.625], [0.25, 0.0]],
                     np.float32)
    for route, gate in ((route2, gate2), (route2[:, :1], np.ones((T, 1), np.float32))):
        got = ref.ffn_moe(x, experts, route, gate)
        for t in range(T):
            want = [Fraction(0)] * D
            for k in range(route.shape[1]):
                w = experts[int(route[t, k])]
                yk, _, _ = frac_ffn([int(v) for v in xf[t]],
                                    *(gen.as_float(w[m]).astype(int).tolist()
                                      for m in ("W1", "W3", "W2T")))
                want = [a + Fraction(float(gate[t, k])) * b for a, b in zip(want, yk)]
            assert [Fraction(v) for v in got[t]] == want


def test_moe_invariants():
    """Relabelling the experts (and the routing with them) leaves y unchanged; with every
    expert the same FFN and gates summing to one, y is that FFN's output."""
    D, H, E, T, K = 32, 48, 5, 7, 2
    experts = [gen.standard_weights(D, H, 0.8, cfg=60, replica=e, dtype="bf16") for e in range(E)]
    x = gen.tokens(D, T, cfg=60, dtype="bf16")
    route, gate = gen.moe_routing(T, E, K, cfg=60)
    base = ref.ffn_moe(x, experts, route, gate)
    perm = np.array([3, 0, 4, 1, 2])                      # new label of expert e is perm[e]
    relabelled = [None] * E
    for e in range(E):
        relabelled[perm[e]] = experts[e]
    np.testing.assert_array_equal(ref.ffn_moe(x, relabelled, perm[route], gate), base)
    same = [experts[0]] * E
    one = ref.ffn_standard(x, experts[0]["W1"], experts[0]["W3"], experts[0]["W2T"])["y"]
    g = np.full((T, K), 0.5, np.float32)
    np.testing.assert_allclose(ref.ffn_moe(x, same, route, g), one, rtol=1e-13, atol=1e-13)
    # route order within a token only reorders the two terms of the sum
    np.testing.assert_allclose(ref.ffn_moe(x, experts, route[:, ::-1], gate[:, ::-1]), base,
                               rtol=1e-13, atol=1e-13)


def test_moe_routing_recipe():
    route, gate = gen.moe_routing(200, 8, 2, cfg=61)
    assert route.dtype == np.int32 and gate.dtype == np.float32 and route.shape == (200, 2)
    assert ((route >= 0) & (route < 8)).all() and (route[:, 0] != route[:, 1]).all()
    assert (gate > 0).all() and np.allclose(gate.sum(axis=1), 1.0, atol=1e-6)
    assert len(np.unique(route)) == 8


def test_dense_equals_sparse_bitwise():
    check_dense_equals_sparse()


def test_all_live_and_none_live():
    check_all_and_none_live()


def test_live_set_monotone_in_offset():
    D, H = 64, 200
    x = gen.tokens(D, 2, cfg=78, dtype="f32")
    prev = None
    for c in np.linspace(-3, 3, 13):
        w = gen.standard_weights(D, H, None, cfg=78, dtype="f32", offset=float(c))
        res = ref.ffn_standard(x, w["W1"], w["W3"], w["W2T"])
        sets = [set(l.tolist()) for l in res["live"]]
        if prev is not None:
            assert all(p <= s for p, s in zip(prev, sets))
        prev = sets


def test_thread_count_does_not_change_results():
    D, H = 512, 1024
    x = gen.tokens(D, 2, cfg=79, dtype="bf16")
    w = gen.standard_weights(D, H, 0.9, cfg=79, dtype="bf16")
    n0 = oracle.num_threads()
    try:
        oracle.set_threads(1)
        a = ref.ffn_standard(x, w["W1"], w["W3"], w["W2T"], act=ref.ACT_RSPLUS)
        oracle.set_threads(max(2, n0))
        b = ref.ffn_standard(x, w["W1"], w["W3"], w["W2T"], act=ref.ACT_RSPLUS)
    finally:
        oracle.set_threads(n0)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["z"], b["z"])


def test_shards_over_hidden_units_sum_to_full_output():
    # splitting the hidden units across devices and summing partial outputs gives y
    D, H, G = 128, 256, 4
    x = gen.tokens(D, 2, cfg=80, dtype="bf16")
    w = gen.standard_weights(D, H, 0.8, cfg=80, dtype="bf16")
    full = ref.ffn_standard(x, w["W1"], w["W3"], w["W2T"])
    acc = np.zeros_like(full["y"])
    for g in range(G):
        sl = slice(g * H // G, (g + 1) * H // G)
        acc += ref.ffn_standard(x, w["W1"][sl], w["W3"][sl], w["W2T"][sl])["y"]
    np.testing.assert_allclose(acc, full["y"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("D,H,s,T,tol", [
    (256, 704, 0.9, 16, 0.015),     # the tiny workload; 11k units, sd of the estimate ~0.3 pt
    (2560, 7168, 0.69, 8, 0.005),
    (2560, 7168, 0.76, 8, 0.005),
    (2560, 7168, 0.896, 8, 0.005),
    (2560, 7168, 0.9, 8, 0.005),
])
def test_sparsity_calibration(D, H, s, T, tol):
    x = gen.tokens(D, T, cfg=2, dtype="bf16" if D > 256 else "f32")
    w = gen.standard_weights(D, H, s, cfg=2, dtype="bf16" if D > 256 else "f32")
    res = ref.ffn_standard(x, w["W1"], w["W3"], w["W2T"], act=ref.ACT_RSPLUS)
    measured = 1.0 - res["k"].sum() / (T * H)
    assert abs(measured - s) <= tol, measured


def test_lopa_sparsity_calibration():
    D, Hp, r = 2560, 9787, 400
    x = gen.tokens(D, 8, cfg=3, dtype="bf16")
    w = gen.lopa_weights(D, Hp, r, 0.9, cfg=3, dtype="bf16")
    res = ref.ffn_lopa(x, w["V"], w["U"], w["W3"], w["W2T"])
    measured = 1.0 - res["k"].sum() / (8 * Hp)
    assert abs(measured - 0.9) <= 0.01, measured
    # V's first row is e_0, so t_0 = x_0 = 1 for every token (the bias rank)
    assert np.all(res["t"][:, 0] == 1.0)


MUTATIONS = {
    "drop_up_projection": ("a[q] = h * (double_act ? orc_activation(act, u) : u);",
                           "a[q] = h * (double_act ? orc_activation(act, u) : 1.0);"),
    "double_act_ignored": ("a[q] = h * (double_act ? orc_activation(act, u) : u);", "a[q] = h * u;"),
    "g_not_tiled": ("double g = (flags & ORC_G_TILED) ? xd[i % D] : 0.0;",
                    "double g = (flags & ORC_G_TILED) ? xd[(i + 1) % D] : 0.0;"),
    "rms_sum_not_mean": ("double inv = 1.0 / sqrt(ss / (double)r + ORC_RMS_EPS);",
                         "double inv = 1.0 / sqrt(ss + ORC_RMS_EPS);"),
    "rms_no_eps": ("double inv = 1.0 / sqrt(ss / (double)r + ORC_RMS_EPS);",
                   "double inv = 1.0 / sqrt(ss / (double)r);"),
    "sigmoid_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "live_test_not_strict": ("z[i] > 0.0", "z[i] >= 0.0"),
    "leaky_relu": ("return z > 0.0 ? z : 0.0;", "return z > 0.0 ? z : 0.01 * z;"),
    "w2_transposed": ("y[j] += aq * elem(W2T, dtype, base + (size_t)j);",
                      "y[j] += aq * elem(W2T, dtype, (size_t)j * (size_t)H + (size_t)vis[q]);"),
    "dot_drops_last_term": ("for (int j = 0; j < n; ++j) s += elem", "for (int j = 0; j + 1 < n; ++j) s += elem"),
    "x_reversed": ("s += elem(M, dtype, base + (size_t)j) * v[j];",
                   "s += elem(M, dtype, base + (size_t)j) * v[n - 1 - j];"),
    "lopa_skips_v": ("for (int m = 0; m < r; ++m) t[m] = dot_row(V, dtype, (size_t)m, D, xd);",
                     "for (int m = 0; m < r; ++m) t[m] = xd[m % D];"),
    "gate_uses_w3": ("for (int i = 0; i < H; ++i) z[i] = dot_row(W1, dtype, (size_t)i, D, xd);",
                     "for (int i = 0; i < H; ++i) z[i] = dot_row(W3, dtype, (size_t)i, D, xd);"),
    "bf16_wrong_shift": ("(uint32_t)((const uint16_t *)p)[idx] << 16;", "(uint32_t)((const uint16_t *)p)[idx] << 15;"),
}
PINS = [check_bruteforce, check_numpy_float, check_rsplus, check_lopa_is_standard_with_uv,
        check_dense_equals_sparse, check_all_and_none_live, check_lopa_full_g_is_materialised_gate,
        check_lopa_full_double_act_exact, check_lopa_full_double_act_reduces_to_single,
        check_lopa_full_rmsnorm]


def _run_pins_with(path_so):
    """Run every pin against another build of the oracle; return the names that fail."""
    caught = []
    with ref.library(path_so):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, RuntimeError):
                caught.append(pin.__name__)
    return caught


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_pins_catch_planted_mistakes():
    src = open(os.path.join(ROOT, "oracle", "sffn_oracle.c")).read()
    with tempfile.TemporaryDirectory() as td:
        for name, (old, new) in MUTATIONS.items():
            assert src.count(old) >= 1, f"mutation {name} does not apply"
            path_c = os.path.join(td, name + ".c")
            path_so = os.path.join(td, name + ".so")
            with open(path_c, "w") as f:
                f.write(src.replace(old, new))
            subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", path_so,
                            path_c, "-lm"], check=True)
            # each planted build runs in a child process so a crash cannot take the suite down
            code = ("import sys; sys.path[:0] = [%r, %r]; import test_oracle as t; "
                    "print('CAUGHT=' + ','.join(t._run_pins_with(%r)))"
                    % (ROOT, os.path.join(ROOT, "tests"), path_so))
            out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                                 timeout=600)
            line = [l for l in out.stdout.splitlines() if l.startswith("CAUGHT=")]
            assert out.returncode == 0 and line, (name, out.returncode, out.stderr[-2000:])
            assert line[0] != "CAUGHT=", f"no pin catches the planted mistake {name!r}"
