"""Sparse attention over shared offsets or per-query edge lists, fp64.

Sources:

* page 1, "Depth-Staggered Fibonacci Spacing for Sparse Attention": the key set
  of query i is the dense window of distances 0..W (self included) plus one
  interpolated key per rung; rung k sits at distance d_k = lo_k + frac_k and is
  the linear interpolation of the rows i - lo_k and i - lo_k - 1 (the two
  integer distances around d_k) of the rotary-rotated keys; values are gathered
  the same way without rotation.  Heads are grouped (GQA, 8 query heads over
  2 key/value heads on that page).
* page 2, "Critical power-law sparse attention", item 2, and page 3,
  "Christoffel-Balanced Sparse Attention", pseudocode: logits Q_i K_j^T/sqrt(d)
  over the allowed keys only, softmax, weighted value sum.

Conventions and readings:

* Every window distance and every rung is its own logit slot, even when two
  slots name the same row (duplicates keep their multiplicity).
* Window slot s is valid iff i - s >= 0; rung k is valid iff i >= d_k, i.e.
  (i - lo_k) >= frac_k.  Signed offsets (page 3, "Christoffel-Balanced
  Sparse Attention": bidirectional attention by signed offsets): a negative
  integer lo_k names the later row i - lo_k = i + |lo_k|, valid iff it is
  below n.  Rows at negative positions are zero (they are only
  ever touched with weight 0, at i = lo_k with frac_k = 0).
* Scale is 1/sqrt(head_dim) unless given.  Query head h uses key/value head
  h // (Hq/Hkv).
* Outputs: o [B, n, Hq, D]; lse [B, Hq, n] = log sum_slots exp(logit).
* The backward differentiates L = <O, dO>.  dd[k] is dL/dd_k inside one
  interpolation cell (the derivative of the rung row pair with respect to the
  distance is row(i-lo-1) - row(i-lo)); dtheta = (alpha-1/2)(3/2-alpha) *
  sum_k f_k dd[k] (chain rule through d_k = alpha f_k and the alpha map).

Layouts: q [B, n, Hq, D]; k, v [B, n, Hkv, D]; everything float64 inside.

transpose_edges and backward_edges (the edge-list backward) are pinned by
brute-force membership checks of the inverted table and by torch autograd
through a dense masked-softmax formulation with rotation.

Pinned by tests/test_oracle_attention.py: torch scaled_dot_product_attention
with an explicit multiplicity mask (integer offsets) and with is_causal (full
window), a per-query loop that builds each interpolated key with numpy.interp,
GQA against repeated-head MHA, central finite differences of the forward for
every gradient, and torch autograd through an explicit dense formulation.
"""

import math

import numpy as np

from . import rope as _rope
from .offsets import dalpha_dtheta


def _shift(x, s):
    """y[:, i] = x[:, i - s] for i - s in [0, n), else 0 (sequence axis 1).
    A negative s reads later rows (signed offsets of bidirectional layers)."""
    y = np.zeros_like(x)
    n = x.shape[1]
    if 0 <= s < n:
        y[:, s:] = x[:, : n - s]
    elif -n < s < 0:
        y[:, : n + s] = x[:, -s:]
    return y


def _unshift(x, s):
    """Adjoint of _shift: y[:, j] = x[:, j + s] for j + s in [0, n), else 0."""
    y = np.zeros_like(x)
    n = x.shape[1]
    if 0 <= s < n:
        y[:, : n - s] = x[:, s:]
    elif -n < s < 0:
        y[:, -s:] = x[:, : n + s]
    return y


def slots(window, lo, frac):
    """Slot list: window distances 0..W then the rungs, as (lo, w, rung)."""
    out = [(s, 0.0, -1) for s in range(window + 1)]
    for k, (l, f) in enumerate(zip(lo, frac)):
        out.append((int(l), float(f), k))
    return out


def _check(q, k, v):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, n, hq, d = q.shape
    if k.shape != v.shape or k.shape[:2] != (B, n) or k.shape[3] != d:
        raise ValueError("shape mismatch")
    hkv = k.shape[2]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return q, k, v, hq // hkv


def _rep(x, g):
    return np.repeat(x, g, axis=2) if g > 1 else x


def _slot_rows(x, lo, w):
    """Interpolated rows (1-w) x[i-lo] + w x[i-lo-1], plus both taps."""
    xa = _shift(x, lo)
    xb = _shift(x, lo + 1)
    return (1.0 - w) * xa + w * xb, xa, xb


def _valid(n, lo, w):
    # the nearer row i - lo must exist: i >= lo + frac, and for a negative
    # (future) offset i - lo <= n - 1
    i = np.arange(n, dtype=np.float64)
    return ((i - lo) >= w) & ((i - lo) <= n - 1)


def _logits(q, k, v, window, lo, frac, rope_base, scale):
    q, k, v, g = _check(q, k, v)
    B, n, hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qr = _rope.rotate(q, rope_base)
    kr = _rope.rotate(k, rope_base)
    sl = slots(window, lo, frac)
    S = np.empty((len(sl), B, n, hq))
    for t, (l, w, _) in enumerate(sl):
        kt, _, _ = _slot_rows(kr, l, w)
        s = np.einsum("bihd,bihd->bih", qr, _rep(kt, g)) * scale
        s[:, ~_valid(n, l, w), :] = -np.inf
        S[t] = s
    return S, qr, kr, v, g, sl, scale


def _softmax(S):
    m = S.max(axis=0)
    e = np.exp(S - m[None])
    l = e.sum(axis=0)
    return e / l[None], m + np.log(l)


def forward(q, k, v, window, lo, frac, rope_base=0.0, scale=None):
    """Causal window-plus-rungs attention.  Returns (o, lse)."""
    S, qr, kr, v, g, sl, scale = _logits(q, k, v, window, lo, frac, rope_base, scale)
    P, lse = _softmax(S)
    o = np.zeros(qr.shape)
    for t, (l, w, _) in enumerate(sl):
        vt, _, _ = _slot_rows(v, l, w)
        o += P[t][..., None] * _rep(vt, g)
    return o, np.transpose(lse, (0, 2, 1)).copy()


def backward(q, k, v, dout, window, lo, frac, rope_base=0.0, scale=None):
    """Gradients of L = <O, dO>: returns dict(dq, dk, dv, dd, o, lse)."""
    S, qr, kr, v, g, sl, scale = _logits(q, k, v, window, lo, frac, rope_base, scale)
    do = np.asarray(dout, dtype=np.float64)
    P, lse = _softmax(S)
    B, n, hq, d = qr.shape
    hkv = hq // g
    vts = []
    o = np.zeros(qr.shape)
    for t, (l, w, _) in enumerate(sl):
        vt, va, vb = _slot_rows(v, l, w)
        vts.append((vt, va, vb))
        o += P[t][..., None] * _rep(vt, g)
    dp = np.stack([np.einsum("bihd,bihd->bih", do, _rep(vt, g)) for vt, _, _ in vts])
    dvec = (P * dp).sum(axis=0)                       # = rowsum(dO * O)
    dS = P * (dp - dvec[None])
    dqr = np.zeros(qr.shape)
    dkr = np.zeros(kr.shape)
    dv = np.zeros(v.shape)
    dd = np.zeros(len(lo))
    for t, (l, w, rung) in enumerate(sl):
        kt, ka, kb = _slot_rows(kr, l, w)
        vt, va, vb = vts[t]
        dqr += scale * dS[t][..., None] * _rep(kt, g)
        # per key/value head: sum over the grouped query heads
        dkt = scale * (dS[t][..., None] * qr).reshape(B, n, hkv, g, d).sum(axis=3)
        dvt = (P[t][..., None] * do).reshape(B, n, hkv, g, d).sum(axis=3)
        dkr += (1.0 - w) * _unshift(dkt, l) + w * _unshift(dkt, l + 1)
        dv += (1.0 - w) * _unshift(dvt, l) + w * _unshift(dvt, l + 1)
        if rung >= 0:
            dd[rung] = np.sum(dkt * (kb - ka)) + np.sum(dvt * (vb - va))
    dq = _rope.rotate_back(dqr, rope_base)
    dk = _rope.rotate_back(dkr, rope_base)
    return {
        "dq": dq,
        "dk": dk,
        "dv": dv,
        "dd": dd,
        "o": o,
        "lse": np.transpose(lse, (0, 2, 1)).copy(),
    }


def dtheta_from_dd(dd, base, alpha):
    """dL/dtheta = (alpha-1/2)(3/2-alpha) * sum_k f_k dd_k."""
    dalpha = 0.0
    for f, x in zip(base, dd):
        dalpha += float(f) * float(x)
    return dalpha_dtheta(alpha) * dalpha


def forward_edges(q, k, v, edges, count, rope_base=0.0, scale=None):
    """Attention over a per-query key list shared by batch and heads.

    edges int[n][width] (ascending, -1 padded), count int[n].  Slot t of
    query i is valid iff t < count[i].  No causal filter (the power-law lists
    are bidirectional).  Returns (o, lse).
    """
    q, k, v, g = _check(q, k, v)
    B, n, hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    edges = np.asarray(edges)
    count = np.asarray(count)
    width = edges.shape[1]
    qr = _rope.rotate(q, rope_base)
    kr = _rope.rotate(k, rope_base)
    S = np.full((width, B, n, hq), -np.inf)
    for t in range(width):
        valid = t < count
        j = np.where(valid, edges[:, t], 0)
        kt = kr[:, j]
        s = np.einsum("bihd,bihd->bih", qr, _rep(kt, g)) * scale
        s[:, ~valid, :] = -np.inf
        S[t] = s
    P, lse = _softmax(S)
    o = np.zeros(qr.shape)
    for t in range(width):
        valid = t < count
        j = np.where(valid, edges[:, t], 0)
        o += P[t][..., None] * _rep(v[:, j], g)
    return o, np.transpose(lse, (0, 2, 1)).copy()


def transpose_edges(edges, count):
    """Inverted edge table for the key-side gather of the edge-list backward.

    For every key j: the slots s = i * width + t with t < count[i] and
    edges[i, t] = j, in ascending (i, t) order.  Returns (inv int[n][cap],
    -1 padded, inv_count int[n]) with cap the largest in-degree (at least 1).
    """
    edges = np.asarray(edges)
    count = np.asarray(count)
    n, width = edges.shape
    lists = [[] for _ in range(n)]
    for i in range(n):
        for t in range(int(count[i])):
            lists[int(edges[i, t])].append(i * width + t)
    cap = max(1, max(len(x) for x in lists)) if n else 1
    inv = np.full((n, cap), -1, dtype=np.int32)
    inv_count = np.zeros(n, dtype=np.int32)
    for j, x in enumerate(lists):
        inv[j, : len(x)] = x
        inv_count[j] = len(x)
    return inv, inv_count


def backward_edges(q, k, v, dout, edges, count, rope_base=0.0, scale=None):
    """Gradients of L = <O, dO> for forward_edges: dict(dq, dk, dv, o, lse).

    Same steps as the shared-offset backward with one plain key per slot:
    dp = dO . v_j, Dvec = sum p dp, dS = p (dp - Dvec), dq~ = scale sum dS
    k~_j, and every slot adds scale dS q~_i to dk~_j and p dO_i to dv_j.
    """
    q, k, v, g = _check(q, k, v)
    B, n, hq, d = q.shape
    hkv = hq // g
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    edges = np.asarray(edges)
    count = np.asarray(count)
    width = edges.shape[1]
    do = np.asarray(dout, dtype=np.float64)
    qr = _rope.rotate(q, rope_base)
    kr = _rope.rotate(k, rope_base)
    keys, valids = [], []
    S = np.full((width, B, n, hq), -np.inf)
    for t in range(width):
        valid = t < count
        j = np.where(valid, edges[:, t], 0)
        keys.append(j)
        valids.append(valid)
        s = np.einsum("bihd,bihd->bih", qr, _rep(kr[:, j], g)) * scale
        s[:, ~valid, :] = -np.inf
        S[t] = s
    P, lse = _softmax(S)
    o = np.zeros(qr.shape)
    dp = np.zeros(S.shape)
    for t in range(width):
        vt = _rep(v[:, keys[t]], g)
        o += P[t][..., None] * vt
        dp[t] = np.einsum("bihd,bihd->bih", do, vt)
    dvec = (P * dp).sum(axis=0)
    dS = P * (dp - dvec[None])
    dqr = np.zeros(qr.shape)
    dkr = np.zeros(kr.shape)
    dv = np.zeros(v.shape)
    for t in range(width):
        j, valid = keys[t], valids[t]
        dqr += scale * dS[t][..., None] * _rep(kr[:, j], g)
        dkt = scale * (dS[t][..., None] * qr).reshape(B, n, hkv, g, d).sum(axis=3)
        dvt = (P[t][..., None] * do).reshape(B, n, hkv, g, d).sum(axis=3)
        iv = np.nonzero(valid)[0]
        np.add.at(dkr, (slice(None), j[iv]), dkt[:, iv])
        np.add.at(dv, (slice(None), j[iv]), dvt[:, iv])
    return {
        "dq": _rope.rotate_back(dqr, rope_base),
        "dk": _rope.rotate_back(dkr, rope_base),
        "dv": dv,
        "o": o,
        "lse": np.transpose(lse, (0, 2, 1)).copy(),
    }
