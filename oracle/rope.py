"""Rotary position embedding in fp64.

Source: page 1 ("Depth-Staggered Fibonacci Spacing for Sparse Attention"),
gather paragraph (rotary embeddings applied at true positions before the
gather) and architecture paragraph (theta_rope = 1e4); the rotary method is
Su et al. (2021), cited in page 1's related-work paragraph.

Reading: interleaved pairs (x[2p], x[2p+1]) are treated as the complex number
x[2p] + i x[2p+1] and multiplied by exp(i * m * theta_p) with
theta_p = base^(-2p/D), where m is the 0-based position in the sequence.
base == 0 means no rotation.  V is never rotated.

Pinned by tests/test_oracle_rope.py (numpy complex multiplication, the
relative-position property, norm preservation).
"""

import numpy as np


def angles(n, head_dim, base):
    """Angle table [n, head_dim/2] in fp64: m * base^(-2p/D)."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    p = np.arange(head_dim // 2, dtype=np.float64)
    inv = np.power(float(base), -2.0 * p / head_dim)
    m = np.arange(n, dtype=np.float64)
    return m[:, None] * inv[None, :]


def rotate(x, base):
    """Rotate x [..., n, H, D] (sequence axis -3) at positions 0..n-1."""
    x = np.asarray(x, dtype=np.float64)
    if not base:
        return x.copy()
    n, d = x.shape[-3], x.shape[-1]
    ang = angles(n, d, base)[:, None, :]          # [n, 1, D/2]
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def rotate_back(x, base):
    """Transpose (inverse) rotation, used for gradients: R(m)^T x."""
    x = np.asarray(x, dtype=np.float64)
    if not base:
        return x.copy()
    n, d = x.shape[-3], x.shape[-1]
    ang = angles(n, d, base)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c + xo * s
    out[..., 1::2] = -xe * s + xo * c
    return out
