"""Pins for oracle.christoffel (page 3: the carry word and its offsets)."""

import json
import os

import pytest

from oracle import christoffel as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("m,k", [(3, 8), (5, 13), (64, 512), (128, 1024),
                                 (0, 7), (7, 7), (1, 1), (37, 100)])
def test_balance_and_count(m, k):
    c = C.carry_word(m, k)
    assert len(c) == k and set(c) <= {0, 1}
    assert sum(c) == m                                   # m ones per period
    # prefix balance: sum_{j<t} c_j = floor(t m / k) (telescoping)
    acc = 0
    for t in range(k + 1):
        assert acc == (t * m) // k
        assert abs(acc - t * m / k) < 1
        if t < k:
            acc += c[t]
    assert C.offsets(m, k) == [j for j in range(k) if c[j]]


def test_hand_derived_words():
    assert "".join(map(str, C.carry_word(3, 8))) == "00100101"
    assert C.carry_word(1, 4) == [0, 0, 0, 1]


def test_page_example_pairs_are_eighths():
    with open(os.path.join(GOLDEN, "christoffel_pairs.json")) as f:
        pairs = json.load(f)["pairs"]
    for m, k in pairs:
        # m/k = 1/8: c[j] = 1 exactly when 8 divides j + 1
        assert C.offsets(m, k) == [8 * q + 7 for q in range(m)]


def test_bad_arguments():
    for m, k in ((-1, 8), (9, 8), (1, 0)):
        with pytest.raises(ValueError):
            C.carry_word(m, k)
