"""The f16 rounding scale of dd (oracle/tolerance.py) against simulated rounding.

The bf16 kernels round dS, p and the rotated queries to f16; the tests bound
the resulting dd error by 4 u L2 with L2 from dd_rounding_scale.  Here the
same roundings are simulated in fp64 on several seeds: every rung's error
must lie inside the bound, and the errors, in units of their predicted
standard deviation u L2 / sqrt(3), must average about one (a scale that is
10x too large or too small fails).
"""

import math

import numpy as np

import synth_inputs as si
from oracle import attention as A
from oracle import offsets
from oracle import tolerance as T


def test_dd_f16_error_inside_rounding_bound_and_at_its_scale():
    ratios = []
    for seed in (1, 2, 3):
        q, k, v = si.qkv(2, 256, 8, 2, 64, "bf16", seed=seed)
        do = si.upstream(2, 256, 8, 64, "bf16", seed=seed)
        f = [si.to_f64(t) for t in (q, k, v, do)]
        alpha = 0.7886
        lo, frac = offsets.rung_offsets(alpha)
        exact = A.backward(*f, 10, lo, frac, 1e4)["dd"]
        l2, dd16 = T.dd_rounding_scale(*f, 10, lo, frac, 1e4)
        err = np.abs(dd16 - exact)
        assert np.all(err <= 4 * T.U16 * l2), (err, 4 * T.U16 * l2)
        live = l2 > 0  # rungs beyond the sequence have no terms at all
        assert live.sum() >= 10 and np.all(exact[~live] == 0)
        ratios.extend(err[live] / (T.U16 * l2[live] / math.sqrt(3)))
    mean = float(np.mean(ratios))
    assert 0.2 < mean < 2.5, mean


def test_dd_f16_is_exact_when_roundings_are_exact():
    # Without rotation and with every rounded quantity already a short binary
    # fraction, the f16 roundings change nothing, so dd_f16 must be the same
    # sum as the oracle's dd.  Keys 0 make every logit 0: with the self slot
    # and one integer rung, a query has one or two valid slots and p is 1 or
    # 1/2; v, dO in {-1, 0, 1} keep dp, Dvec and dS (scale 1/2 at d = 4)
    # multiples of 1/4.
    n, d = 12, 4
    rng = np.random.default_rng(0)
    q = rng.integers(-1, 2, size=(1, n, 1, d)).astype(np.float64)
    k = np.zeros((1, n, 1, d))
    v = rng.integers(-1, 2, size=(1, n, 1, d)).astype(np.float64)
    do = rng.integers(-1, 2, size=(1, n, 1, d)).astype(np.float64)
    lo = np.array([3], dtype=np.int32)
    frac = np.array([0.0], dtype=np.float32)
    exact = A.backward(q, k, v, do, 0, lo, frac, 0.0)["dd"]
    _, dd16 = T.dd_rounding_scale(q, k, v, do, 0, lo, frac, 0.0)
    assert exact[0] != 0
    assert np.allclose(dd16, exact, rtol=0, atol=1e-12), (dd16, exact)
