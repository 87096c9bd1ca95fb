"""Work counters against the figures the pages print (CPU only)."""
import json
import math
import os
from fractions import Fraction as F

from oracle import counts as c

from conftest import GOLDEN


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def trunc1(x):
    return math.floor(x * 10) / 10


def test_fig2_per_matrix_macs():
    g = load("fig2_macs.json")
    D, H, r, Hp, s = g["D"], g["H"], g["r"], g["H_prime"], F(str(g["sparsity"]))
    p = g["printed_millions"]
    assert c.macs_per_matrix_dense(D, H) == 18_350_080
    assert trunc1(c.macs_per_matrix_dense(D, H) / 1e6) == p["dense_per_matrix"]
    sparse_w = (1 - s) * H * D            # one skippable matrix at sparsity s
    assert sparse_w == 1_835_008
    assert trunc1(float(sparse_w) / 1e6) == p["sparse_w3"] == p["sparse_w2"]
    gate = c.macs_lopa(D, Hp, r, 0)
    assert gate == 4_938_800
    assert trunc1(gate / 1e6) == p["lopa_gate"]
    lopa_w = (1 - s) * Hp * D
    assert lopa_w == F(2_505_472)
    assert trunc1(float(lopa_w) / 1e6) == p["lopa_w3"] == p["lopa_w2"]
    # the sparse counters reproduce the same totals at k = (1-s) H
    k = int((1 - s) * H)
    assert c.macs_sparse(D, H, k) == 18_350_080 + 2 * 1_835_008 - 2 * D * 0 - 2 * D * ((1 - s) * H - k)


def test_hidden_width_matches_fig2():
    g = load("fig2_macs.json")
    Hp = c.hidden_width_lopa(g["D"], g["H"], g["r"])
    assert 9787 < Hp < 9788
    assert c.hidden_width_lopa_int(g["D"], g["H"], g["r"]) == g["H_prime"]
    # H' keeps the parameter count: exact at the unfloored width, 2000 short at the floor
    assert c.params_lopa(g["D"], Hp, g["r"]) == c.params_standard(g["D"], g["H"])
    assert c.params_standard(g["D"], g["H"]) - c.params_lopa(g["D"], g["H_prime"], g["r"]) == 2000


def test_eq2_points_and_limit():
    g = load("flop_ratios.json")["eq2"]
    for s, printed, tol in g["points"]:
        assert abs(float(c.flop_ratio_standard(F(str(s)))) - printed) <= tol
    # the general form 3HD / (HD + 2(1-s)HD) reduces to 3/(3-2s) for any H, D
    for (D, H) in [(2560, 7168), (7, 11)]:
        s = F(9, 10)
        direct = F(c.macs_dense(D, H)) / (H * D + 2 * (1 - s) * H * D)
        assert direct == c.flop_ratio_standard(s)
    # monotone, tends to 3 and never reaches it
    vals = [c.flop_ratio_standard(F(i, 100)) for i in range(0, 100)]
    assert all(a < b for a, b in zip(vals, vals[1:]))
    assert c.flop_ratio_standard(1) == g["limit"]
    assert c.flop_ratio_standard(0) == 1


def test_widget_lopa_shares_and_speedup():
    g = load("flop_ratios.json")["widget"]
    D = F(1)
    H = F(*g["H_over_D"]) * D
    r = F(*g["r_over_D"]) * D
    s = F(str(g["sparsity"]))
    sh = c.lopa_shares(D, H, r, s)
    pct = g["percent_of_dense"]
    assert round(float(sh["gate"]) * 100, 1) == pct["gate"]
    assert round(float(sh["w3"]) * 100, 1) == pct["w3"]
    assert round(float(sh["w2"]) * 100, 1) == pct["w2"]
    assert round(float(sh["total"]) * 100) == pct["total"]
    sp = float(c.flop_ratio_lopa(D, H, r, s))
    assert abs(sp - g["speedup"]) <= g["speedup_tol"]
    assert abs(sp - 1 / float(sh["total"])) < 1e-12
    lim = float(c.flop_ratio_lopa(D, H, r, 1))
    assert abs(lim - g["limit_about"]) <= g["limit_tol"]
    assert abs(lim - 13.6) < 1e-12


def test_standard_table_speedups():
    for p in load("flop_ratios.json")["tables_standard"]["points"]:
        s, hw = F(str(p["s"])), F(str(p["s_halfwidth"]))
        lo = float(c.flop_ratio_standard(s - hw))
        hi = float(c.flop_ratio_standard(s + hw))
        q = 10 ** -p["digits"] / 2
        # some sparsity inside the printed rounding interval rounds to the printed speedup
        assert lo - q <= p["speedup"] <= hi + q, (p, lo, hi)


def test_lopa_ratio_at_fig2_shape():
    # at the Figure 2 shape the LoPA FFN reads 5.53x fewer weights than the dense one at s = 0.9
    D, H, r, Hp = 2560, 7168, 400, 9787
    k = F(1, 10) * Hp
    ratio = F(c.macs_dense(D, H)) / (r * (D + Hp) + 2 * k * D)
    assert abs(float(ratio) - 5.533) < 5e-4
    assert c.touched_bytes(c.macs_dense(D, H)) == 2 * 3 * H * D
