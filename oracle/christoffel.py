"""Christoffel carry word and its offset set, in exact integer arithmetic.

Source: "Christoffel-Balanced Sparse Attention" (page 3), the construction and
its pseudocode: c[j] = floor((j+1) m / k) - floor(j m / k) for j = 0..k-1, the
allowed offsets are the positions j with c[j] == 1.

Reading for the causal kernel (the page's pseudocode adds the offset and then
keeps only keys at or before the query, which would drop every positive
offset): offsets are backward distances, the key of query i at offset o is
row i - o, valid when i - o >= 0.  One period (o < k) is used.  The query's
own row is added as the distance-0 window slot, as on page 1.

Pinned by tests/test_oracle_christoffel.py (exactly m ones per period, the
telescoping prefix-sum closed form, hand-derived words).
"""


def carry_word(m, k):
    """The 0/1 word c[0..k-1]; requires 0 <= m <= k and k >= 1."""
    if k < 1 or m < 0 or m > k:
        raise ValueError("need k >= 1 and 0 <= m <= k")
    return [((j + 1) * m) // k - (j * m) // k for j in range(k)]


def offsets(m, k):
    """O = { j : c[j] == 1 }, ascending."""
    return [j for j, c in enumerate(carry_word(m, k)) if c == 1]


def signed_offsets(m, k):
    """Bidirectional offset set of page 3 ("signed offsets"): -O and +O,
    ascending (keys i + o and i - o for every o in O)."""
    o = offsets(m, k)
    return sorted([-x for x in o] + o)
