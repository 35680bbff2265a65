"""sfa_bwd_noalloc (the backward with the library's static scratch as its
workspace) against sfa_bwd with a caller workspace, through the C ABI: two
calls in a row on one device, the second smaller, each bit-identical to
sfa_bwd's results (the same kernels run on the same inputs)."""

import ctypes

import numpy as np
import pytest
import torch

import synth_inputs as si

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _sfa():
    import fixed_offset_gather_amd as sfa
    return sfa


def _both(B, n, hq, hkv, D, dtype, W, alpha, seed):
    sfa = _sfa()
    q, k, v = (t.to(DEV) for t in si.qkv(B, n, hq, hkv, D, dtype, seed))
    do = si.upstream(B, n, hq, D, dtype, seed).to(DEV)
    rope = sfa.rope_table_device(n, D, 1e4, DEV)
    lo, fr = sfa.offsets_fib(alpha)
    base = sfa.base_fib()
    o, lse = sfa.fwd(q, k, v, W, lo, fr, rope, want_lse=True)
    ref = sfa.bwd(q, k, v, lse, do, W, lo, fr, rope, base=base, alpha=alpha)
    pr = sfa.Problem(q, k, W, lo, fr, rope)
    assert sfa.library().sfa_bwd_workspace_bytes(pr.ref()) <= sfa.NOALLOC_SCRATCH_BYTES
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dd = torch.empty(len(lo), dtype=torch.float32, device=DEV)
    dth = torch.empty(1, dtype=torch.float32, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = sfa.library().sfa_bwd_noalloc(pr.ref(), p(q), p(k), p(v), p(lse), p(do), p(dq), p(dk), p(dv), p(dd),
                                       base.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), float(alpha), p(dth),
                                       stream)
    assert rc == 0, sfa.library().sfa_last_error()
    torch.cuda.synchronize()
    return ref, (dq, dk, dv, dd, dth)


def test_noalloc_matches_sfa_bwd_twice_second_smaller():
    alpha = si.learned_alpha()
    print("call 1: page-1 layer shape, 4 x 1024, 8/2 heads, bf16, W 10, alpha %.6f" % alpha, flush=True)
    ref, got = _both(4, 1024, 8, 2, 64, "bf16", 10, alpha, si.SEED)
    for name, a, b in zip(("dq", "dk", "dv", "dd", "dtheta"), ref, got):
        assert torch.equal(a, b), name
    print("call 2: 2 x 200, 4/2 heads, head dim 32, fp32, W 3, alpha 0.713", flush=True)
    ref, got = _both(2, 200, 4, 2, 32, "f32", 3, 0.713, 7)
    for name, a, b in zip(("dq", "dk", "dv", "dd", "dtheta"), ref, got):
        assert torch.equal(a, b), name
    assert np.isfinite(got[4].item())
