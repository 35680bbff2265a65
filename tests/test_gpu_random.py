"""Seeded random configurations of the shared-offset path, on the GPU,
through the C ABI, against the oracle at the stated tolerances.

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
