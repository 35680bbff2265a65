"""Rounding scale of the offset gradient for 16-bit operands (test infrastructure).

Not part of the method: this module sizes the error that the bf16 kernels'
own arithmetic puts into dd_k, so the tests can bound it.

dd_k (page 1, "Depth-Staggered Fibonacci Spacing for Sparse Attention",
gather paragraph: the interpolated row keeps a gradient to the distance) is a
sum over every (query, head, dim) of elementary products

    scale dS q~_d (k~b_d - k~a_d)      and      p dO_d (vb_d - va_d)

with k~a, k~b (va, vb) the floor and floor-plus-one rows.  The bf16 kernels
round each dS and p (one per query and head) and each rotated query element
q~_d to f16 before multiplying, accumulating in fp32.  A rounding to f16
changes a value by a relative amount of at most u = 2^-11, spread about
evenly over [-u, u] (standard deviation u / sqrt(3)), independently from one
rounded value to the next.  The first-order error of dd_k is therefore a sum
of independent terms whose size is set by

    L2_k = sqrt( sum_{i,h} (scale dS (q~ . dk~))^2
               + sum_{i,h,d} (scale dS q~_d dk~_d)^2
               + sum_{i,h} (p (dO . dv))^2 ),

one entry per rounded value, and its standard deviation is (u / sqrt 3) L2_k.
The tests allow 4 u L2_k (about 7 standard deviations).  When dd_k is a near
cancellation of large terms this is the binding bound; otherwise the plain
relative bound is.

dd_f16 simulates exactly those roundings (numpy float16 rounds to nearest
even, as the kernels' conversions do) in fp64 otherwise, so a CPU test can
check that the bound covers them.
"""

import numpy as np

from . import attention as _att

U16 = 2.0 ** -11  # unit roundoff of IEEE half precision


def dd_rounding_scale(q, k, v, dout, window, lo, frac, rope_base=0.0, scale=None):
    """(L2 [K], dd_f16 [K]) for the shared-offset attention's K rungs."""
    S, qr, kr, vv, g, sl, scale = _att._logits(q, k, v, window, lo, frac, rope_base, scale)
    do = np.asarray(dout, dtype=np.float64)
    P, _ = _att._softmax(S)
    B, n, hq, d = qr.shape
    vts = [_att._slot_rows(vv, l, w) for l, w, _ in sl]
    dp = np.stack([np.einsum("bihd,bihd->bih", do, _att._rep(vt, g)) for vt, _, _ in vts])
    dvec = (P * dp).sum(axis=0)
    dS = P * (dp - dvec[None])
    f16 = lambda x: np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)
    qr16 = f16(qr)
    l2 = np.zeros(len(lo))
    dd16 = np.zeros(len(lo))
    for t, (l, w, rung) in enumerate(sl):
        if rung < 0:
            continue
        _, ka, kb = _att._slot_rows(kr, l, w)
        _, va, vb = vts[t]
        dk = _att._rep(kb - ka, g)
        dv = _att._rep(vb - va, g)
        ws = scale * dS[t]
        tk = ws[..., None] * qr * dk                     # [B, n, hq, d]
        tv = P[t][..., None] * do * dv
        l2[rung] = np.sqrt((tk.sum(axis=-1) ** 2).sum() + (tk ** 2).sum() + (tv.sum(axis=-1) ** 2).sum())
        dd16[rung] = ((f16(ws)[..., None] * qr16 * dk).sum()
                      + (f16(P[t])[..., None] * f16(do) * dv).sum())
    return l2, dd16
