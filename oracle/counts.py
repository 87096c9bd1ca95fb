"""Exact work counters for the gated FFN (test infrastructure only).

Counts are multiply-adds (MACs), the unit in which the pages count "FLOPs":
one matrix of the FFN costs H*D of them per token (page "Model casting: compute
the gate, then skip most of the FFN", section "What an FFN actually
computes"). Everything is integer or Fraction arithmetic so the printed
figures can be checked exactly.

* dense:    3 H D                                 (same section)
* sparse:   H D + 2 k D                           (section "The 3x ceiling, and why
                                                   W1 is always on": W1 always runs,
                                                   W3 rows and W2 columns only for live units)
* LoPA:     r (D + H') + 2 k D                    (section "LoPA Gating: moving the
                                                   ceiling": the low-rank gate costs r(D + H'))
* Eq. 2:    3HD / (HD + 2(1-s)HD) = 3 / (3 - 2s)
* H':       D (3H - r) / (r + 2D), the hidden width that keeps the parameter
            count of a LoPA FFN equal to the standard one (same section);
            the paper card's Figure 2 prints the floor, 9787, for
            D = 2560, H = 7168, r = 400.
* Eq. 4:    3HD / (r (D + H') + 2 (1-s) H' D), the LoPA FLOP ratio, obtained by
            putting the LoPA gate cost into the Eq. 2 ratio as that section does.
"""
from __future__ import annotations

from fractions import Fraction
import math


def macs_dense(D: int, H: int) -> int:
    return 3 * H * D


def macs_sparse(D: int, H: int, k: int) -> int:
    return H * D + 2 * k * D


def macs_lopa(D: int, Hp: int, r: int, k: int) -> int:
    return r * (D + Hp) + 2 * k * D


def macs_per_matrix_dense(D: int, H: int) -> int:
    return H * D


def hidden_width_lopa(D, H, r) -> Fraction:
    """H' = D (3H - r) / (r + 2D), exact."""
    return Fraction(D) * (3 * Fraction(H) - Fraction(r)) / (Fraction(r) + 2 * Fraction(D))


def hidden_width_lopa_int(D: int, H: int, r: int) -> int:
    return math.floor(hidden_width_lopa(D, H, r))


def params_standard(D: int, H: int) -> int:
    return 3 * H * D


def params_lopa(D: int, Hp: int, r: int) -> int:
    """U (H' x r) + V (r x D) + W3 (H' x D) + W2 (D x H')."""
    return r * (Hp + D) + 2 * Hp * D


def flop_ratio_standard(s) -> Fraction:
    """Eq. 2 with the dense cost over the sparse cost, as a Fraction of s."""
    s = Fraction(s)
    return Fraction(3) / (3 - 2 * s)


def flop_ratio_lopa(D, H, r, s, Hp=None) -> Fraction:
    """Eq. 4: 3HD / (r (D + H') + 2 (1-s) H' D); H' exact unless given."""
    s = Fraction(s)
    D, H, r = Fraction(D), Fraction(H), Fraction(r)
    Hp = hidden_width_lopa(D, H, r) if Hp is None else Fraction(Hp)
    return 3 * H * D / (r * (D + Hp) + 2 * (1 - s) * Hp * D)


def lopa_shares(D, H, r, s, Hp=None) -> dict:
    """Fractions of a dense FFN's MACs spent on the LoPA gate, W3 and W2."""
    s = Fraction(s)
    D, H, r = Fraction(D), Fraction(H), Fraction(r)
    Hp = hidden_width_lopa(D, H, r) if Hp is None else Fraction(Hp)
    dense = 3 * H * D
    gate = r * (D + Hp) / dense
    w3 = (1 - s) * Hp * D / dense
    return {"gate": gate, "w3": w3, "w2": w3, "total": gate + 2 * w3}


def touched_bytes(macs: int, bytes_per_weight: int = 2) -> int:
    """Weight bytes read for a MAC count: one weight per multiply-add."""
    return macs * bytes_per_weight
