"""Power-law per-query edge lists (fixed-degree sampling).

Source: "Critical power-law sparse attention" (page 2), items 1-2: always keep
a local window of radius r, then m times draw a distance d from
q(d) = d^-(1+sigma) / sum_{u=1}^{floor(n/2)} u^-(1+sigma), draw a random sign,
add j = (i + s d) mod n, and deduplicate.

The page fixes no random generator, so the sampler is specified here and
implemented independently on the library side from the same text:

* mix(x) is SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): add the golden
  gamma 0x9E3779B97F4A7C15, then two xor-shift-multiply rounds and a final
  xor-shift, all modulo 2^64.
* Query i uses key_i = mix(seed XOR mix(i)); draw t uses a = mix(key_i + 2t)
  and b = mix(key_i + 2t + 1).
* u = (a >> 11) * 2^-53 in [0, 1); d is the smallest d in [1, floor(n/2)] with
  u < CDF[d], where CDF[d] is the prefix sum of v^-(1+sigma) over v <= d
  (accumulated in increasing v, fp64) divided by the full sum, and
  CDF[floor(n/2)] is set to 1.
* sign = +1 when the top bit of b is 0, else -1.

Readings: the window is clipped to [0, n) (not wrapped); the long-range keys
wrap modulo n as written; the list is the sorted union, padded with -1 to the
table width.  One table serves every batch entry and head.

Pinned by tests/test_oracle_powerlaw.py (SplitMix64 reference outputs, the
normaliser against the Hurwitz zeta function, a chi-square test of drawn
distances against q(d), structural invariants).
"""

import bisect

import numpy as np

_MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def mix(x):
    """SplitMix64 output for generator state x (state advanced by gamma first)."""
    z = (x + _GAMMA) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def distance_cdf(n, sigma):
    """CDF of q(d) over d = 1..floor(n/2) (list index d-1), fp64."""
    half = n // 2
    if half < 1:
        raise ValueError("need n >= 2")
    expo = -(1.0 + float(sigma))
    weights = [float(v) ** expo for v in range(1, half + 1)]
    z = 0.0
    for w in weights:
        z += w
    cdf = []
    acc = 0.0
    for w in weights:
        acc += w
        cdf.append(acc / z)
    cdf[-1] = 1.0
    return cdf


def draw_distance(u, cdf):
    """Smallest d (1-based) with u < CDF[d]."""
    return bisect.bisect_right(cdf, u) + 1


def query_draws(i, seed, draws, cdf):
    """The (distance, sign) pairs drawn for query i."""
    key = mix((seed ^ mix(i)) & _MASK64)
    out = []
    for t in range(draws):
        a = mix((key + 2 * t) & _MASK64)
        b = mix((key + 2 * t + 1) & _MASK64)
        u = (a >> 11) * (2.0 ** -53)
        d = draw_distance(u, cdf)
        s = 1 if (b >> 63) == 0 else -1
        out.append((d, s))
    return out


def edge_lists(n, r, sigma, draws, width, seed):
    """Edge table int32[n][width] (ascending, -1 padded) and count int32[n]."""
    if n < 2 or r < 0 or draws < 0 or width < 1:
        raise ValueError("bad arguments")
    cdf = distance_cdf(n, sigma)
    edges = np.full((n, width), -1, dtype=np.int32)
    count = np.zeros(n, dtype=np.int32)
    for i in range(n):
        nb = set(range(max(0, i - r), min(n, i + r + 1)))
        for d, s in query_draws(i, seed, draws, cdf):
            nb.add((i + s * d) % n)
        row = sorted(nb)
        if len(row) > width:
            raise ValueError("edge list of query %d exceeds the table width" % i)
        edges[i, : len(row)] = row
        count[i] = len(row)
    return edges, count
