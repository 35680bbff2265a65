"""Rung bases, the alpha map, per-layer schedules and rung offsets (fp64).

Source: "Depth-Staggered Fibonacci Spacing for Sparse Attention" (page 1):
the fib equation (K = 15 rungs), the gather paragraph (d_k = alpha * f_k;
a fractional distance lerps the two rows whose distances bracket it), the alpha
parameterisation (alpha = 0.5 + sigmoid(theta)), the schedule list (fixed,
learned, staggered linear, staggered coprime with S = 7 over L = 16 layers)
and the reach-matched power-of-2 control.

Readings where the page leaves a step open:

* The rung distance is the fp64 product ``alpha * f`` (one rounding); the row
  pair is ``lo = floor(d)`` and ``lo + 1``, the weight of the farther row is
  ``frac = d - lo`` (exact in fp64) stored as float32.
* The linear ramp value ``0.5 + s/(L-1)`` is the correctly rounded fp64 of the
  exact rational ``(2s + L - 1) / (2(L - 1))``.  Summing ``0.5 + s/15`` in two
  roundings would misplace floors (e.g. s = 5, f = 144 gives 119.999...).
* Coprime stagger: layer l receives the ramp value of index ``(S*l) mod L``.
* Power-of-2 control base: ``2^0 .. 2^10`` (K = 11; 1024 is the power of two
  that matches the Fibonacci reach 987 ~ 1024 the page itself equates).

Pinned by tests/test_oracle_offsets.py (page list, exact rationals, closed
forms, numeric derivative of the alpha map).
"""

from fractions import Fraction
import math

import numpy as np

# The page-1 fib equation.
FIB_BASE = (1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987)

# Reach-matched log-sparse control (reading stated in the module docstring).
POW2_BASE = tuple(1 << e for e in range(11))

SCHEDULES = ("fixed", "linear", "coprime")


def alpha_of_theta(theta):
    """alpha = 0.5 + sigmoid(theta)  (page 1, alpha parameterisation)."""
    theta = float(theta)
    return 0.5 + 1.0 / (1.0 + math.exp(-theta))


def theta_of_alpha(alpha):
    """Inverse of the alpha map on the open interval (0.5, 1.5)."""
    alpha = float(alpha)
    if not (0.5 < alpha < 1.5):
        raise ValueError("alpha must lie strictly inside (0.5, 1.5)")
    return math.log((alpha - 0.5) / (1.5 - alpha))


def dalpha_dtheta(alpha):
    """sigmoid'(theta) written through alpha: (alpha - 1/2)(3/2 - alpha)."""
    alpha = float(alpha)
    return (alpha - 0.5) * (1.5 - alpha)


def ramp_alpha(s, L):
    """Linear ramp value 0.5 + s/(L-1), exact rational rounded once to fp64."""
    if L < 2 or not (0 <= s < L):
        raise ValueError("need L >= 2 and 0 <= s < L")
    return float(Fraction(1, 2) + Fraction(s, L - 1))


def schedule_alpha(kind, layer, L=16, S=7):
    """Per-layer alpha for the three static schedules of page 1.

    fixed:   1 for every layer.
    linear:  0.5 + l/(L-1).
    coprime: the linear multiset reassigned, layer l gets index (S*l) mod L.
    """
    if not (0 <= layer < L):
        raise ValueError("layer out of range")
    if kind == "fixed":
        return 1.0
    if kind == "linear":
        return ramp_alpha(layer, L)
    if kind == "coprime":
        if math.gcd(S, L) != 1:
            raise ValueError("stride must be coprime with L")
        return ramp_alpha((S * layer) % L, L)
    raise ValueError("unknown schedule %r" % (kind,))


def rung_offsets(alpha, base=FIB_BASE):
    """Scaled rungs d_k = alpha * f_k split into (lo_k, frac_k).

    Returns (lo int32[K], frac float32[K]).  K = len(base).
    """
    alpha = float(alpha)
    if not (math.isfinite(alpha) and alpha > 0.0):
        raise ValueError("alpha must be finite and positive")
    lo = np.empty(len(base), dtype=np.int32)
    frac = np.empty(len(base), dtype=np.float32)
    for k, f in enumerate(base):
        d = alpha * float(f)           # one fp64 rounding
        fl = math.floor(d)
        lo[k] = fl
        frac[k] = np.float32(d - fl)   # exact subtraction, then to float32
    return lo, frac
