"""Pins for oracle.offsets against what page 1 and exact arithmetic fix."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import offsets as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_fib_base_is_the_page_list():
    with open(os.path.join(GOLDEN, "fibonacci_base.json")) as f:
        g = json.load(f)
    assert list(O.FIB_BASE) == g["values"]
    assert len(O.FIB_BASE) == g["K"] == 15
    # Fibonacci recurrence and the reach the page compares with 1024.
    for a, b, c in zip(O.FIB_BASE, O.FIB_BASE[1:], O.FIB_BASE[2:]):
        assert a + b == c
    assert O.FIB_BASE[-1] == 987


def test_pow2_control_reach_and_count():
    assert O.POW2_BASE[0] == 1 and O.POW2_BASE[-1] == 1024
    assert len(O.POW2_BASE) < len(O.FIB_BASE)  # fewer rungs at matched reach
    assert all(b == 2 * a for a, b in zip(O.POW2_BASE, O.POW2_BASE[1:]))


def test_alpha_map_init_range_and_derivative():
    assert O.alpha_of_theta(0.0) == 1.0              # learned init: alpha = 1
    for th in (-30.0, -3.0, -0.5, 0.7, 4.0, 30.0):
        a = O.alpha_of_theta(th)
        assert 0.5 <= a <= 1.5
    for th in (-2.0, -0.3, 0.0, 0.9, 2.5):
        h = 1e-5
        num = (O.alpha_of_theta(th + h) - O.alpha_of_theta(th - h)) / (2 * h)
        assert abs(num - O.dalpha_dtheta(O.alpha_of_theta(th))) < 1e-9
        assert abs(O.theta_of_alpha(O.alpha_of_theta(th)) - th) < 1e-12


def test_linear_schedule_ramp():
    L = 16
    vals = [O.schedule_alpha("linear", l, L) for l in range(L)]
    assert vals[0] == 0.5 and vals[-1] == 1.5
    for l, a in enumerate(vals):
        assert a == float(Fraction(1, 2) + Fraction(l, L - 1))
    assert all(O.schedule_alpha("fixed", l, L) == 1.0 for l in range(L))


def test_coprime_schedule_permutation():
    L, S = 16, 7
    # (7 l) mod 16 evaluated by hand for l = 0..15
    perm = [0, 7, 14, 5, 12, 3, 10, 1, 8, 15, 6, 13, 4, 11, 2, 9]
    lin = [O.schedule_alpha("linear", l, L) for l in range(L)]
    cop = [O.schedule_alpha("coprime", l, L, S) for l in range(L)]
    assert cop == [lin[p] for p in perm]
    assert sorted(cop) == sorted(lin)                     # same multiset
    assert [perm[p] for p in perm] == list(range(L))      # involution
    gaps = {abs(perm[l + 1] - perm[l]) for l in range(L - 1)}
    assert gaps == {7, 9}
    with pytest.raises(ValueError):
        O.schedule_alpha("coprime", 1, 16, 4)


def _exact_split(alpha, f):
    d = Fraction(alpha) * f
    lo = math.floor(d)
    return lo, d - lo


@pytest.mark.parametrize("base", [O.FIB_BASE, O.POW2_BASE])
def test_rung_floors_exact_under_every_schedule(base):
    L = 16
    for kind in O.SCHEDULES:
        for l in range(L):
            a = O.schedule_alpha(kind, l, L)
            lo, frac = O.rung_offsets(a, base)
            ra = Fraction(2 * ((7 * l) % L if kind == "coprime" else l) + L - 1,
                          2 * (L - 1)) if kind != "fixed" else Fraction(1)
            for k, f in enumerate(base):
                d = ra * f                                   # exact rational
                assert lo[k] == math.floor(d), (kind, l, f)
                assert abs(float(frac[k]) - float(d - math.floor(d))) <= 1e-7


def test_exact_integer_rungs_have_zero_frac():
    # distances that are exact integers under the 16-layer ramp (s, f, d)
    cases = [(0, 2, 1), (0, 8, 4), (0, 34, 17), (0, 144, 72), (0, 610, 305),
             (3, 610, 427), (5, 144, 120), (6, 610, 549), (9, 610, 671),
             (10, 144, 168), (12, 610, 793), (15, 2, 3), (15, 8, 12),
             (15, 34, 51), (15, 144, 216), (15, 610, 915)]
    found = []
    for s in range(16):
        a = O.ramp_alpha(s, 16)
        lo, frac = O.rung_offsets(a, O.FIB_BASE)
        for k, f in enumerate(O.FIB_BASE):
            if Fraction(2 * s + 15, 30) * f == int(Fraction(2 * s + 15, 30) * f):
                found.append((s, f, int(lo[k])))
                assert frac[k] == 0.0
    assert found == cases


def test_alpha_one_and_three_quarters():
    lo, frac = O.rung_offsets(1.0)
    assert list(lo) == list(O.FIB_BASE) and not frac.any()
    lo, frac = O.rung_offsets(0.75)
    for k, f in enumerate(O.FIB_BASE):
        l, r = _exact_split(0.75, f)
        assert lo[k] == l and frac[k] == float(r)   # quarters are exact
    assert list(lo) == [0, 1, 2, 3, 6, 9, 15, 25, 41, 66, 108, 174, 282, 457, 740]


def test_rung_offsets_reject_bad_alpha():
    for a in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            O.rung_offsets(a)
    assert O.rung_offsets(1.0)[0].dtype == np.int32
