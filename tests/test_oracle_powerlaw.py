"""Pins for oracle.powerlaw (page 2, items 1-2: power-law edge lists)."""

import numpy as np
import pytest
from scipy import special, stats

from oracle import powerlaw as P


def test_splitmix64_reference_outputs():
    # First four outputs of the SplitMix64 reference generator seeded with 0
    # (Vigna's public-domain splitmix64.c): state += gamma, then the mix.
    gamma = 0x9E3779B97F4A7C15
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
            0x06C45D188009454F, 0xF88BB8A8724C81EC]
    got = [P.mix((t * gamma) & ((1 << 64) - 1)) for t in range(4)]
    assert got == want


def test_normaliser_matches_hurwitz_zeta():
    n, sigma = 2048, 0.8
    cdf = P.distance_cdf(n, sigma)
    s = 1.0 + sigma
    z = special.zeta(s, 1) - special.zeta(s, n // 2 + 1)
    q1 = 1.0 / z
    assert abs(cdf[0] - q1) < 1e-12
    assert len(cdf) == n // 2 and cdf[-1] == 1.0
    assert all(a < b for a, b in zip(cdf, cdf[1:]))
    # probability mass up to d = 8 from the closed form
    p8 = (special.zeta(s, 1) - special.zeta(s, 9)) / z
    assert abs(cdf[7] - p8) < 1e-12


def test_inverse_cdf_boundaries():
    cdf = P.distance_cdf(16, 0.8)
    assert P.draw_distance(0.0, cdf) == 1
    assert P.draw_distance(np.nextafter(cdf[0], 0.0), cdf) == 1
    assert P.draw_distance(cdf[0], cdf) == 2        # u < CDF[d] is strict
    assert P.draw_distance(np.nextafter(1.0, 0.0), cdf) == 8


def test_drawn_distances_follow_the_power_law():
    n, sigma, draws = 2048, 0.8, 47
    cdf = P.distance_cdf(n, sigma)
    ds, signs = [], []
    for i in range(400):
        for d, s in P.query_draws(i, 42, draws, cdf):
            ds.append(d)
            signs.append(s)
    ds = np.array(ds)
    edges = [1, 2, 3, 4, 5, 6, 7, 8, 9, 17, 65, 257, n // 2 + 1]
    obs = np.histogram(ds, bins=edges)[0]
    s = 1.0 + sigma
    z = special.zeta(s, 1) - special.zeta(s, n // 2 + 1)
    expect = np.array([(special.zeta(s, a) - special.zeta(s, b)) / z
                       for a, b in zip(edges[:-1], edges[1:])]) * len(ds)
    assert stats.chisquare(obs, expect).pvalue > 1e-3
    # the random sign is fair
    plus = sum(1 for x in signs if x > 0)
    assert stats.binomtest(plus, len(signs), 0.5).pvalue > 1e-3


@pytest.mark.parametrize("n,r,draws,width", [(256, 4, 20, 32), (2048, 8, 47, 64),
                                             (7, 1, 5, 8)])
def test_edge_table_structure(n, r, draws, width):
    edges, count = P.edge_lists(n, r, 0.8, draws, width, seed=42)
    assert edges.shape == (n, width) and count.shape == (n,)
    for i in range(n):
        c = int(count[i])
        row = edges[i, :c]
        assert 1 <= c <= min(width, 2 * r + 1 + draws)
        assert np.all(np.diff(row) > 0)                   # sorted, unique
        assert np.all((row >= 0) & (row < n))
        assert np.all(edges[i, c:] == -1)
        win = set(range(max(0, i - r), min(n, i + r + 1)))
        assert win <= set(row.tolist())                  # window kept
    if n >= 256:
        # long-range edges reach both directions
        assert (edges[n // 2] > n // 2 + r).any() and (
            (edges[n // 2] >= 0) & (edges[n // 2] < n // 2 - r)).any()


def test_edge_table_deterministic_and_seeded():
    a = P.edge_lists(128, 2, 0.8, 10, 16, seed=1)
    b = P.edge_lists(128, 2, 0.8, 10, 16, seed=1)
    c = P.edge_lists(128, 2, 0.8, 10, 16, seed=2)
    assert np.array_equal(a[0], b[0]) and not np.array_equal(a[0], c[0])


def test_width_too_small_is_an_error():
    with pytest.raises(ValueError):
        P.edge_lists(64, 8, 0.8, 30, 8, seed=0)
