"""Pins for oracle.attention against library routines, brute force and calculus."""

import math

import numpy as np
import pytest
import torch
from scipy import special

from oracle import attention as A
from oracle import christoffel, offsets, powerlaw


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _rope_complex(x, base):
    """Independent rotation through numpy complex numbers."""
    if not base:
        return x.copy()
    n, d = x.shape[1], x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    th = base ** (-2.0 * np.arange(d // 2) / d)
    z = z * np.exp(1j * np.arange(n)[None, :, None, None] * th)
    out = np.empty_like(x)
    out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


def _sdpa(qr, kr, v, mask, g):
    """torch SDPA (fp64, CPU) with an additive float mask [n, n]."""
    q = torch.from_numpy(qr).permute(0, 2, 1, 3)
    k = torch.from_numpy(np.repeat(kr, g, axis=2)).permute(0, 2, 1, 3)
    vv = torch.from_numpy(np.repeat(v, g, axis=2)).permute(0, 2, 1, 3)
    m = torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, vv, attn_mask=m)
    return o.permute(0, 2, 1, 3).numpy()


def _multiplicity(n, window, lo, frac):
    C = np.zeros((n, n))
    for i in range(n):
        for s in range(window + 1):
            if i - s >= 0:
                C[i, i - s] += 1
        for l, f in zip(lo, frac):
            assert f == 0.0
            if i - l >= 0:
                C[i, i - l] += 1
    return C


def _logmask(C):
    with np.errstate(divide="ignore"):
        return np.log(C)


@pytest.mark.parametrize("g", [1, 2])
def test_integer_offsets_match_sdpa_with_multiplicity_mask(g):
    B, n, hkv, d, W = 2, 48, 2, 8, 3
    q, k, v = _rand((B, n, hkv * g, d), 1), _rand((B, n, hkv, d), 2), _rand((B, n, hkv, d), 3)
    lo, frac = offsets.rung_offsets(1.0)
    o, lse = A.forward(q, k, v, W, lo, frac, rope_base=1e4)
    qr, kr = _rope_complex(q, 1e4), _rope_complex(k, 1e4)
    C = _multiplicity(n, W, lo, frac)
    ref = _sdpa(qr, kr, v, _logmask(C), g)
    assert np.abs(o - ref).max() < 1e-12
    # lse: logsumexp of (scaled logit + log multiplicity) over all rows
    s = np.einsum("bihd,bjhd->bhij", qr, np.repeat(kr, g, axis=2)) / math.sqrt(d)
    want = special.logsumexp(s + _logmask(C)[None, None], axis=-1)
    assert np.abs(lse - want).max() < 1e-12


def test_full_window_is_causal_attention():
    B, n, h, d = 1, 33, 2, 16
    q, k, v = _rand((B, n, h, d), 4), _rand((B, n, h, d), 5), _rand((B, n, h, d), 6)
    o, _ = A.forward(q, k, v, n - 1, [], [], rope_base=1e4)
    qt = torch.from_numpy(_rope_complex(q, 1e4)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(_rope_complex(k, 1e4)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    assert np.abs(o - ref.permute(0, 2, 1, 3).numpy()).max() < 1e-12


def test_gqa_equals_repeated_heads():
    B, n, d, W = 1, 40, 8, 2
    q, k, v = _rand((B, n, 4, d), 7), _rand((B, n, 1, d), 8), _rand((B, n, 1, d), 9)
    lo, frac = offsets.rung_offsets(0.75)
    o1, l1 = A.forward(q, k, v, W, lo, frac, 1e4)
    o2, l2 = A.forward(q, np.repeat(k, 4, 2), np.repeat(v, 4, 2), W, lo, frac, 1e4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("alpha", [0.75, 0.7, 1.3])
def test_interpolated_rungs_match_numpy_interp_brute_force(alpha):
    B, n, hq, hkv, d, W = 1, 40, 2, 1, 8, 2
    q, k, v = _rand((B, n, hq, d), 10), _rand((B, n, hkv, d), 11), _rand((B, n, hkv, d), 12)
    lo, frac = offsets.rung_offsets(alpha)
    o, lse = A.forward(q, k, v, W, lo, frac, 1e4)
    qr, kr = _rope_complex(q, 1e4), _rope_complex(k, 1e4)
    pos = np.arange(n, dtype=np.float64)
    for h in range(hq):
        hk = h // (hq // hkv)
        for i in range(n):
            keys, vals = [], []
            for s in range(W + 1):
                if i - s >= 0:
                    keys.append(kr[0, i - s, hk]); vals.append(v[0, i - s, hk])
            for l, f in zip(lo, frac):
                dist = float(l) + float(f)
                if i >= dist:
                    x = i - dist
                    keys.append(np.array([np.interp(x, pos, kr[0, :, hk, c]) for c in range(d)]))
                    vals.append(np.array([np.interp(x, pos, v[0, :, hk, c]) for c in range(d)]))
            logit = np.array(keys) @ qr[0, i, h] / math.sqrt(d)
            p = special.softmax(logit)
            assert np.abs(p @ np.array(vals) - o[0, i, h]).max() < 1e-12
            assert abs(special.logsumexp(logit) - lse[0, h, i]) < 1e-12


def test_integer_alpha_interpolation_is_exact_gather():
    # frac = 0 must reproduce the plain integer gather bit for bit.
    B, n, d = 1, 64, 8
    q, k, v = _rand((B, n, 2, d), 13), _rand((B, n, 1, d), 14), _rand((B, n, 1, d), 15)
    lo, frac = offsets.rung_offsets(1.0)
    o1, _ = A.forward(q, k, v, 4, lo, frac, 1e4)
    C = _multiplicity(n, 4, lo, frac)
    o2 = _sdpa(_rope_complex(q, 1e4), _rope_complex(k, 1e4), v, _logmask(C), 2)
    assert np.abs(o1 - o2).max() < 1e-12


def test_christoffel_through_window_zero():
    B, n, h, d = 1, 70, 1, 8
    q, k, v = _rand((B, n, h, d), 16), _rand((B, n, h, d), 17), _rand((B, n, h, d), 18)
    offs = christoffel.offsets(3, 8)            # [2, 5, 7]
    lo = np.array(offs, dtype=np.int32)
    frac = np.zeros(len(offs), dtype=np.float32)
    o, _ = A.forward(q, k, v, 0, lo, frac, 0.0)
    C = np.zeros((n, n))
    for i in range(n):
        C[i, i] = 1
        for oo in offs:
            if i - oo >= 0:
                C[i, i - oo] = 1
    assert np.abs(o - _sdpa(q, k, v, _logmask(C), 1)).max() < 1e-12


def test_edge_lists_match_sdpa_with_boolean_mask():
    B, n, h, d = 2, 64, 2, 8
    q, k, v = _rand((B, n, h, d), 19), _rand((B, n, h, d), 20), _rand((B, n, h, d), 21)
    edges, count = powerlaw.edge_lists(n, 2, 0.8, 6, 16, seed=5)
    o, lse = A.forward_edges(q, k, v, edges, count)
    M = np.full((n, n), -np.inf)
    for i in range(n):
        M[i, edges[i, : count[i]]] = 0.0
    assert np.abs(o - _sdpa(q, k, v, M, 1)).max() < 1e-12
    s = np.einsum("bihd,bjhd->bhij", q, k) / math.sqrt(d)
    assert np.abs(lse - special.logsumexp(s + M, axis=-1)).max() < 1e-12


# ---------------------------------------------------------------- gradients

def _loss(q, k, v, do, W, lo, frac, base):
    o, _ = A.forward(q, k, v, W, lo, frac, base)
    return float(np.sum(o * do))


def _case(alpha=0.713, n=26):
    B, hq, hkv, d, W = 2, 4, 2, 8, 2
    q, k, v = _rand((B, n, hq, d), 30), _rand((B, n, hkv, d), 31), _rand((B, n, hkv, d), 32)
    do = _rand((B, n, hq, d), 33)
    lo, frac = offsets.rung_offsets(alpha)
    return q, k, v, do, W, lo, frac


def test_backward_matches_finite_differences():
    q, k, v, do, W, lo, frac = _case()
    g = A.backward(q, k, v, do, W, lo, frac, 1e4)
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        u = _rand(x.shape, 99)
        args = {"dq": 0, "dk": 1, "dv": 2}[name]
        xp, xm = [q, k, v], [q, k, v]
        xp = [a + eps * u if i == args else a for i, a in enumerate(xp)]
        xm = [a - eps * u if i == args else a for i, a in enumerate(xm)]
        num = (_loss(*xp, do, W, lo, frac, 1e4) - _loss(*xm, do, W, lo, frac, 1e4)) / (2 * eps)
        ana = float(np.sum(g[name] * u))
        assert abs(num - ana) < 1e-7 * max(1.0, abs(ana)), name
    # one derivative per rung distance, inside its interpolation cell
    for kk in range(len(lo)):
        fp, fm = frac.astype(np.float64).copy(), frac.astype(np.float64).copy()
        fp[kk] += eps
        fm[kk] -= eps
        num = (_loss(q, k, v, do, W, lo, fp, 1e4) - _loss(q, k, v, do, W, lo, fm, 1e4)) / (2 * eps)
        assert abs(num - g["dd"][kk]) < 1e-7 * max(1.0, abs(num)), kk


def test_dtheta_matches_finite_difference_in_theta():
    alpha = 0.713          # every alpha * f_k is at least 0.02 from an integer
    q, k, v, do, W, lo, frac = _case(alpha)
    g = A.backward(q, k, v, do, W, lo, frac, 1e4)
    th = offsets.theta_of_alpha(alpha)
    ana = A.dtheta_from_dd(g["dd"], offsets.FIB_BASE, alpha)
    h = 1e-7

    def L(theta):
        a = offsets.alpha_of_theta(theta)
        d = [a * f for f in offsets.FIB_BASE]
        l = np.floor(d).astype(np.int32)
        assert np.array_equal(l, lo)          # the step stays inside every cell
        return _loss(q, k, v, do, W, l, np.array(d) - l, 1e4)

    num = (L(th + h) - L(th - h)) / (2 * h)
    assert abs(num - ana) < 1e-6 * max(1.0, abs(ana))


def _dense_torch_forward(q, k, v, W, lo, frac, base):
    """Explicit slot matrices A_i applied to dense tensors (torch, fp64)."""
    B, n, hq, d = q.shape
    hkv = k.shape[2]
    g = hq // hkv
    th = base ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    ang = torch.arange(n, dtype=torch.float64)[:, None] * th[None]
    rot = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]

    def rope(x):
        z = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
        return torch.view_as_real(z * rot).reshape(x.shape)

    qr, kr = rope(q), rope(k)
    outs = []
    for i in range(n):
        rows = []
        for s in range(W + 1):
            if i - s >= 0:
                e = torch.zeros(n, dtype=torch.float64); e[i - s] = 1.0; rows.append(e)
        for l, f in zip(lo, frac):
            if i - l >= f:
                e = torch.zeros(n, dtype=torch.float64)
                e[i - l] += 1.0 - float(f)
                if i - l - 1 >= 0:
                    e[i - l - 1] += float(f)
                rows.append(e)
        Ai = torch.stack(rows)                                  # [S_i, n]
        heads = []
        for h in range(hq):
            kt = Ai @ kr[:, :, h // g, :]                       # [B, S_i, d]
            vt = Ai @ v[:, :, h // g, :]
            logit = torch.einsum("bsd,bd->bs", kt, qr[:, i, h]) / math.sqrt(d)
            p = torch.softmax(logit, dim=-1)
            heads.append(torch.einsum("bs,bsd->bd", p, vt))
        outs.append(torch.stack(heads, dim=1))
    return torch.stack(outs, dim=1)


def test_backward_matches_autograd_of_dense_formulation():
    q, k, v, do, W, lo, frac = _case(alpha=0.75, n=20)
    g = A.backward(q, k, v, do, W, lo, frac, 1e4)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    o = _dense_torch_forward(tq, tk, tv, W, lo, frac, 1e4)
    assert np.abs(o.detach().numpy() - g["o"]).max() < 1e-12
    (o * torch.from_numpy(do)).sum().backward()
    assert np.abs(tq.grad.numpy() - g["dq"]).max() < 1e-11
    assert np.abs(tk.grad.numpy() - g["dk"]).max() < 1e-11
    assert np.abs(tv.grad.numpy() - g["dv"]).max() < 1e-11


# ------------------------------------------------------- edge-list backward

def _torch_rope(x, base):
    d, n = x.shape[-1], x.shape[1]
    th = base ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    ang = torch.arange(n, dtype=torch.float64)[:, None] * th[None]
    rot = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]
    z = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
    return torch.view_as_real(z * rot).reshape(x.shape)


def test_transpose_edges_brute_force():
    n = 90
    edges, count = powerlaw.edge_lists(n, 3, 0.8, 9, 20, seed=7)
    inv, inv_count = A.transpose_edges(edges, count)
    width = edges.shape[1]
    assert inv_count.sum() == count.sum()
    for j in range(n):
        row = inv[j, : inv_count[j]]
        assert np.all(np.diff(row) > 0) and np.all(inv[j, inv_count[j]:] == -1)
        for s in row:
            i, t = divmod(int(s), width)
            assert t < count[i] and edges[i, t] == j
    for i in range(n):
        for t in range(count[i]):
            assert i * width + t in inv[edges[i, t], : inv_count[edges[i, t]]]


def test_edge_backward_matches_autograd_of_dense_masked_attention():
    # Bidirectional lists that include the query itself, GQA 4/2, RoPE.
    B, n, hq, hkv, d = 2, 40, 4, 2, 8
    q, k, v, do = (_rand((B, n, h, d), s) for h, s in ((hq, 31), (hkv, 32), (hkv, 33), (hq, 34)))
    edges, count = powerlaw.edge_lists(n, 2, 0.8, 5, 12, seed=3)
    g = A.backward_edges(q, k, v, do, edges, count, 1e4)
    M = torch.full((n, n), -math.inf, dtype=torch.float64)
    for i in range(n):
        M[i, torch.from_numpy(edges[i, : count[i]].astype(np.int64))] = 0.0
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    qr, kr = _torch_rope(tq, 1e4), _torch_rope(tk, 1e4)
    kr2, v2 = kr.repeat_interleave(hq // hkv, dim=2), tv.repeat_interleave(hq // hkv, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", qr, kr2) / math.sqrt(d) + M
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), v2)
    assert np.abs(o.detach().numpy() - g["o"]).max() < 1e-12
    (o * torch.from_numpy(do)).sum().backward()
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert np.abs(t.grad.numpy() - g[name]).max() < 1e-11, name
    o2, lse2 = A.forward_edges(q, k, v, edges, count, 1e4)
    assert np.abs(o2 - g["o"]).max() < 1e-13 and np.abs(lse2 - g["lse"]).max() < 1e-13


# ------------------------------------------------ signed (bidirectional) offsets

def test_signed_offsets_forward_and_backward_match_dense_masked_attention():
    # Bidirectional Christoffel (self + signed carry-word offsets, page 3):
    # keys i - o and i + o inside [0, n); GQA 4/2 with rotation.
    B, n, hq, hkv, d = 2, 48, 4, 2, 8
    q, k, v, do = (_rand((B, n, h, d), s) for h, s in ((hq, 41), (hkv, 42), (hkv, 43), (hq, 44)))
    offs = np.array(christoffel.signed_offsets(4, 16), dtype=np.int32)
    assert list(offs[:4]) == [-15, -11, -7, -3] and list(offs[4:]) == [3, 7, 11, 15]
    fr = np.zeros(len(offs))
    g = A.backward(q, k, v, do, 0, offs, fr, 1e4)
    M = torch.full((n, n), -math.inf, dtype=torch.float64)
    for i in range(n):
        for o in [0] + list(offs):
            if 0 <= i - o < n:
                M[i, i - o] = 0.0
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    qr, kr = _torch_rope(tq, 1e4), _torch_rope(tk, 1e4)
    kr2, v2 = kr.repeat_interleave(hq // hkv, dim=2), tv.repeat_interleave(hq // hkv, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", qr, kr2) / math.sqrt(d) + M
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), v2)
    assert np.abs(o.detach().numpy() - g["o"]).max() < 1e-12
    (o * torch.from_numpy(do)).sum().backward()
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert np.abs(t.grad.numpy() - g[name]).max() < 1e-11, name


def test_signed_interpolated_offset_dd_matches_finite_difference():
    # A negative offset inside an interpolation cell: rows i + 5 (weight
    # 0.7) and i + 4 (0.3); dd by central differences in frac.
    B, n, h, d = 1, 30, 2, 8
    q, k, v, do = (_rand((B, n, h, d), s) for s in (51, 52, 53, 54))
    lo = np.array([-5, 3], dtype=np.int32)
    fr = np.array([0.3, 0.6])
    g = A.backward(q, k, v, do, 1, lo, fr, 1e4)
    eps = 1e-6
    for kk in range(2):
        fp, fm = fr.copy(), fr.copy()
        fp[kk] += eps
        fm[kk] -= eps
        num = (_loss(q, k, v, do, 1, lo, fp, 1e4) - _loss(q, k, v, do, 1, lo, fm, 1e4)) / (2 * eps)
        assert abs(num - g["dd"][kk]) < 1e-7 * max(1.0, abs(num)), kk
