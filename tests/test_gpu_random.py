"""Seeded random configurations of every key set, on the GPU, through the C
ABI, against the oracle at the stated tolerances: shared offsets (below),
power-law edge lists and signed (bidirectional) offsets (further below), and
shared offsets at head dim 128 (bf16, last).

Each case draws its own shape and offset table: fp32 or bf16; 1, 2, 4 or 8
query heads per KV head over one or two KV heads; head dim 16, 32 or 64; one
or two sequences of 1 to 260 tokens (ragged against every block size); a
window of 0 to 16; 0 to 24 rungs at alpha times a random increasing integer
base (alpha in [0.55, 1.45], so most rungs are interpolated and some land on
integers); RoPE 1e4 or none; the offset gradient on or off.  The forward
(O, LSE) and the backward (dQ, dK, dV, and dd, dtheta when asked) are checked
with the same bounds as the fixed parity cases: max abs error <= 1e-5 for
fp32 tensors, <= 1e-2 beyond the output's own rounding for bf16, and dd,
dtheta within tol * max(1, |ref|).  The draws are fixed by the seed, so a
failure names a reproducible case.
"""

import numpy as np
import pytest

import test_gpu_parity as P

pytestmark = pytest.mark.gpu

N_CASES = 48
SEED = 2027


def _draw(idx):
    rng = np.random.default_rng(SEED + 7919 * idx)
    dtype = ["f32", "bf16"][int(rng.integers(2))]
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.integers(1, 3))
    D = int(rng.choice([16, 32, 64]))
    B = int(rng.integers(1, 3))
    n = int(rng.integers(1, 261))
    W = int(rng.integers(0, 17))
    n_rungs = int(rng.integers(0, 25))
    base = np.sort(rng.choice(np.arange(1, max(2 * n, 4) + 1), size=min(n_rungs, max(2 * n, 4)), replace=False))
    alpha = float(rng.uniform(0.55, 1.45))
    theta = [1e4, 0.0][int(rng.integers(2))]
    want_dd = bool(rng.integers(2)) and len(base) > 0
    return dict(dtype=dtype, hq=G * hkv, hkv=hkv, D=D, B=B, n=n, W=W, base=base.astype(np.int32), alpha=alpha,
                theta=theta, want_dd=want_dd, seed=int(rng.integers(1, 10_000)))


@pytest.mark.parametrize("idx", range(N_CASES))
def test_random_configuration(idx):
    c = _draw(idx)
    sfa = P._sfa()
    lo, frac = sfa.offsets_scaled(c["base"], c["alpha"])
    print("case %d: %s" % (idx, {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in c.items()}),
          flush=True)
    case = P.Case(c["B"], c["n"], c["hq"], c["hkv"], c["D"], c["dtype"], seed=c["seed"], rope_theta=c["theta"])
    P._fwd_check(case, c["W"], lo, frac)
    P._bwd_check(case, c["W"], lo, frac, c["alpha"], c["base"], want_dd=c["want_dd"])


N_EDGE_CASES = 24
N_SIGNED_CASES = 24


def _draw_edges(idx):
    rng = np.random.default_rng(SEED + 104729 + 7919 * idx)
    dtype = ["f32", "bf16"][int(rng.integers(2))]
    G = int(rng.choice([1, 2, 4]))
    hkv = int(rng.integers(1, 3))
    D = int(rng.choice([16, 32, 64]))
    n = int(rng.integers(2, 301))
    r = int(rng.integers(0, 5))
    draws = int(rng.integers(0, 21))
    width = min(64, 2 * r + 1 + draws + int(rng.integers(0, 9)))
    return dict(dtype=dtype, hq=G * hkv, hkv=hkv, D=D, B=int(rng.integers(1, 3)), n=n, r=r,
                sigma=float(rng.uniform(0.5, 1.5)), draws=draws, width=width, theta=[1e4, 0.0][int(rng.integers(2))],
                edge_seed=int(rng.integers(0, 1 << 30)), seed=int(rng.integers(1, 10_000)))


@pytest.mark.parametrize("idx", range(N_EDGE_CASES))
def test_random_edge_lists(idx):
    # Power-law edge lists (window radius 0-4, 0-20 draws, width up to 64)
    # over random shapes: forward and backward against the oracle.
    c = _draw_edges(idx)
    sfa = P._sfa()
    print("edge case %d: %s" % (idx, c), flush=True)
    edges, count = sfa.edges_powerlaw(c["n"], c["r"], c["sigma"], c["draws"], c["width"], c["edge_seed"])
    case = P.Case(c["B"], c["n"], c["hq"], c["hkv"], c["D"], c["dtype"], seed=c["seed"], rope_theta=c["theta"])
    P._edge_bwd_check(case, edges, count)


def _draw_signed(idx):
    rng = np.random.default_rng(SEED + 1299709 + 7919 * idx)
    dtype = ["f32", "bf16"][int(rng.integers(2))]
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.integers(1, 3))
    n = int(rng.integers(1, 231))
    k = int(rng.integers(1, 25))
    d = np.sort(rng.uniform(-1.5 * n - 2, 1.5 * n + 2, size=k))
    if rng.integers(2):
        d = np.round(d)  # integer distances, some negative
    lo = np.floor(d).astype(np.int32)
    frac = np.minimum((d - lo).astype(np.float32), np.float32(1.0 - 2.0 ** -24))  # below 1 after rounding
    return dict(dtype=dtype, hq=G * hkv, hkv=hkv, D=int(rng.choice([16, 32, 64])), B=int(rng.integers(1, 3)), n=n,
                W=int(rng.integers(0, 12)), lo=lo, frac=frac, base=rng.integers(1, 50, size=k).astype(np.int32),
                alpha=float(rng.uniform(0.6, 1.4)), theta=[1e4, 0.0][int(rng.integers(2))],
                want_dd=bool(rng.integers(2)), seed=int(rng.integers(1, 10_000)))


@pytest.mark.parametrize("idx", range(N_SIGNED_CASES))
def test_random_signed_offsets(idx):
    # Offsets on both sides of the query (a negative offset names the later
    # row i - lo), interpolated or integer, with the causal window, through
    # SFA_FLAG_SIGNED_OFFSETS; the dtheta check takes an arbitrary base and
    # alpha (it is the chain rule through the fractions either way).
    c = _draw_signed(idx)
    print("signed case %d: %s" % (idx, {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in c.items()}),
          flush=True)
    case = P.Case(c["B"], c["n"], c["hq"], c["hkv"], c["D"], c["dtype"], seed=c["seed"], rope_theta=c["theta"])
    P._fwd_check(case, c["W"], c["lo"], c["frac"], signed=True)
    P._bwd_check(case, c["W"], c["lo"], c["frac"], c["alpha"], c["base"], want_dd=c["want_dd"], signed=True)


N_D128_CASES = 16


def _draw_d128(idx):
    # bf16 only (fp32 is refused at head dim 128)
    rng = np.random.default_rng(SEED + 15485863 + 7919 * idx)
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.integers(1, 3))
    n = int(rng.integers(1, 221))
    n_rungs = int(rng.integers(0, 17))
    base = np.sort(rng.choice(np.arange(1, max(2 * n, 4) + 1), size=min(n_rungs, max(2 * n, 4)), replace=False))
    alpha = float(rng.uniform(0.55, 1.45))
    return dict(dtype="bf16", hq=G * hkv, hkv=hkv, D=128, B=int(rng.integers(1, 3)), n=n, W=int(rng.integers(0, 13)),
                base=base.astype(np.int32), alpha=alpha, theta=[1e4, 0.0][int(rng.integers(2))],
                want_dd=bool(rng.integers(2)) and len(base) > 0, seed=int(rng.integers(1, 10_000)))


@pytest.mark.parametrize("idx", range(N_D128_CASES))
def test_random_head_dim_128(idx):
    c = _draw_d128(idx)
    sfa = P._sfa()
    lo, frac = sfa.offsets_scaled(c["base"], c["alpha"])
    print("d128 case %d: %s" % (idx, {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in c.items()}),
          flush=True)
    case = P.Case(c["B"], c["n"], c["hq"], c["hkv"], c["D"], c["dtype"], seed=c["seed"], rope_theta=c["theta"])
    P._fwd_check(case, c["W"], lo, frac)
    P._bwd_check(case, c["W"], lo, frac, c["alpha"], c["base"], want_dd=c["want_dd"])
