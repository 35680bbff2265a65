"""C-ABI library: loads, exports every declared symbol, host producers are
bit-exact against the oracle, and every invalid argument is rejected before
any device call (these tests run without a GPU)."""

import ctypes
import os
import re

import numpy as np
import pytest

import fixed_offset_gather_amd as sfa
from oracle import attention as ref_att
from oracle import christoffel as ref_chr
from oracle import offsets as ref_off
from oracle import powerlaw as ref_pl
from oracle import rope as ref_rope

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "sfa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(sfa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 19
    lib = sfa.library()
    for nm in names:
        assert hasattr(lib, nm), nm
    assert lib.sfa_version() == 1


def test_bases_match_oracle():
    assert list(sfa.base_fib()) == list(ref_off.FIB_BASE)
    assert list(sfa.base_pow2()) == list(ref_off.POW2_BASE)


def _alphas():
    out = [1.0, 0.75, 0.5, 1.5, 0.713, 0.999999, 1.000001, 7.3]
    for kind in ref_off.SCHEDULES:
        for l in range(16):
            out.append(ref_off.schedule_alpha(kind, l, 16, 7))
    rng = np.random.default_rng(0)
    out += list(0.5 + rng.random(200))
    return out


def test_offsets_bit_exact_against_oracle():
    for a in _alphas():
        for lib_fn, base in ((sfa.offsets_fib, ref_off.FIB_BASE), (sfa.offsets_pow2, ref_off.POW2_BASE)):
            lo, frac = lib_fn(a)
            rlo, rfrac = ref_off.rung_offsets(a, base)
            assert np.array_equal(lo, rlo), a
            assert np.array_equal(frac.view(np.uint32), rfrac.view(np.uint32)), a


def test_schedules_bit_exact_against_oracle():
    for kind in ref_off.SCHEDULES:
        for l in range(16):
            assert sfa.stagger_alpha(kind, l, 16, 7) == ref_off.schedule_alpha(kind, l, 16, 7)
    for L, S in ((8, 3), (5, 2), (12, 5)):
        for l in range(L):
            assert sfa.stagger_alpha("coprime", l, L, S) == ref_off.schedule_alpha("coprime", l, L, S)
    for th in (-4.0, -0.3, 0.0, 0.5, 3.0):
        a, d = sfa.alpha_of_theta(th)
        assert a == ref_off.alpha_of_theta(th)
        assert d == ref_off.dalpha_dtheta(a)


@pytest.mark.parametrize("m,k", [(128, 1024), (64, 512), (3, 8), (5, 13), (0, 9), (9, 9), (37, 100),
                                 (1000, 4096)])
def test_christoffel_bit_exact(m, k):
    assert list(sfa.offsets_christoffel(m, k)) == ref_chr.offsets(m, k)


@pytest.mark.parametrize("n,r,sigma,draws,width,seed",
                         [(2048, 8, 0.8, 47, 64, 42), (257, 3, 0.5, 20, 32, 7), (2, 0, 0.8, 3, 4, 1),
                          (1024, 4, 1.2, 30, 48, 123456789012345)])
def test_powerlaw_edges_bit_exact(n, r, sigma, draws, width, seed):
    e, c = sfa.edges_powerlaw(n, r, sigma, draws, width, seed)
    re_, rc = ref_pl.edge_lists(n, r, sigma, draws, width, seed)
    assert np.array_equal(e, re_) and np.array_equal(c, rc)


def test_rope_table_matches_oracle_angles():
    n, d = 1024, 64
    t = sfa.rope_table(n, d, 1e4)
    ang = ref_rope.angles(n, d, 1e4)
    assert np.abs(t[..., 0] - np.cos(ang)).max() < 1.2e-7
    assert np.abs(t[..., 1] - np.sin(ang)).max() < 1.2e-7


# ---------------------------------------------------------- error handling

def _prob(**kw):
    d = dict(batch=1, seqlen=64, hq=8, hkv=2, head_dim=64, dtype=sfa.SFA_BF16, window=8, n_off=0,
             scale=0.0, flags=0)
    d.update(kw)
    lo = np.asarray(kw.pop("lo", []), dtype=np.int32)
    fr = np.asarray(kw.pop("frac", []), dtype=np.float32)
    d.pop("lo", None)
    d.pop("frac", None)
    a = sfa.SfaAttn()
    for key, val in d.items():
        setattr(a, key, val)
    a.n_off = len(lo) if "n_off" not in kw else kw["n_off"]
    a.off_lo = lo.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if len(lo) else None
    a.off_frac = fr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)) if len(fr) else None
    a._keep = (lo, fr)
    return a


FAKE = ctypes.c_void_p(0x100000)       # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x100008)


def _fwd(a, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None):
    lib = sfa.library()
    return lib.sfa_fwd(ctypes.byref(a) if a is not None else None, q, k, v, o, lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(hq=6, hkv=4), sfa.SFA_ERR_ARG),
    (dict(hq=0), sfa.SFA_ERR_ARG),
    (dict(hq=16, hkv=1), sfa.SFA_ERR_UNSUPPORTED),
    (dict(head_dim=128, dtype=sfa.SFA_F32), sfa.SFA_ERR_UNSUPPORTED),
    (dict(head_dim=256), sfa.SFA_ERR_UNSUPPORTED),
    (dict(head_dim=48), sfa.SFA_ERR_UNSUPPORTED),
    (dict(dtype=7), sfa.SFA_ERR_ARG),
    (dict(window=-1), sfa.SFA_ERR_ARG),
    (dict(window=319, lo=[1], frac=[0.0]), sfa.SFA_ERR_UNSUPPORTED),
    (dict(lo=list(range(257)), frac=[0.0] * 257), sfa.SFA_ERR_UNSUPPORTED),
    (dict(lo=[1, -2], frac=[0.0, 0.0]), sfa.SFA_ERR_ARG),
    (dict(lo=[1], frac=[1.0]), sfa.SFA_ERR_ARG),
    (dict(lo=[1], frac=[float("nan")]), sfa.SFA_ERR_ARG),
    (dict(scale=float("nan")), sfa.SFA_ERR_ARG),
    (dict(scale=-1.0), sfa.SFA_ERR_ARG),
    (dict(flags=4), sfa.SFA_ERR_ARG),
    (dict(batch=-1), sfa.SFA_ERR_ARG),
])
def test_fwd_rejects_invalid_problem(kw, code):
    assert _fwd(_prob(**kw)) == code
    assert sfa.library().sfa_last_error()


def test_fwd_rejects_bad_pointers_before_any_device_call():
    a = _prob()
    assert _fwd(None) == sfa.SFA_ERR_ARG
    assert _fwd(a, q=None) == sfa.SFA_ERR_ARG
    assert _fwd(a, o=MISALIGNED) == sfa.SFA_ERR_ARG
    assert _fwd(a, lse=MISALIGNED) == sfa.SFA_ERR_ARG
    lib = sfa.library()
    assert lib.sfa_fwd_edges(ctypes.byref(a), FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, None, None) == sfa.SFA_ERR_ARG
    assert lib.sfa_fwd_edges(ctypes.byref(a), None, FAKE, 8, FAKE, FAKE, FAKE, FAKE, None, None) == sfa.SFA_ERR_ARG


def test_empty_problem_is_a_no_op():
    assert _fwd(_prob(batch=0), q=None, k=None, v=None, o=None) == sfa.SFA_OK
    assert _fwd(_prob(seqlen=0), q=None, k=None, v=None, o=None) == sfa.SFA_OK


def test_bwd_validation_and_workspace_size():
    lib = sfa.library()
    lo, frac = sfa.offsets_fib(0.8)
    a = _prob(batch=2, seqlen=100, lo=lo, frac=frac, window=10)
    nb = lib.sfa_bwd_workspace_bytes(ctypes.byref(a))
    S = 10 + 1 + 15
    al = lambda e: (e + 63) // 64 * 64
    pe = al(2 * 2 * S * 100 * 4)          # p and dp: [B][Hkv][S][n][G]
    de = al(2 * 2 * 100 * 4)              # Dvec / l and 1 / l: [B][Hkv][n][G] each
    # dd partials: one per query-pass workgroup (16-query blocks at 4 heads
    # per KV head, x B x Hkv)
    blocks = 7 * 2 * 2
    dd = al(blocks * 15)
    # packed key-pass rows of q and dO (bf16, G >= 2): D * G / 2 words per row
    xe = al(2 * 2 * 100 * 64 * 2)
    # bounds on |dS| (bf16, G >= 2): one per query-pass workgroup
    we = al(blocks)
    assert nb == (2 * pe + 2 * de + dd + 2 * xe + we) * 4
    assert lib.sfa_bwd_workspace_bytes(ctypes.byref(_prob(head_dim=48))) == 0
    base = sfa.base_fib()
    bp = base.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    args = [FAKE] * 8
    # workspace too small
    rc = lib.sfa_bwd(ctypes.byref(a), *args, None, bp, 0.8, None, FAKE, nb - 4, None)
    assert rc == sfa.SFA_ERR_CAPACITY
    # dtheta without the base
    rc = lib.sfa_bwd(ctypes.byref(a), *args, None, None, 0.8, FAKE, FAKE, nb, None)
    assert rc == sfa.SFA_ERR_ARG
    # null tensor
    rc = lib.sfa_bwd(ctypes.byref(a), *([None] + args[1:]), None, bp, 0.8, None, FAKE, nb, None)
    assert rc == sfa.SFA_ERR_ARG


def test_producer_errors():
    lib = sfa.library()
    out = np.zeros(4, dtype=np.int32)
    p = out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert lib.sfa_base_fib(p, 4) == sfa.SFA_ERR_CAPACITY
    assert lib.sfa_offsets_christoffel(8, 4, p, 4) == sfa.SFA_ERR_ARG
    assert lib.sfa_offsets_christoffel(5, 8, p, 4) == sfa.SFA_ERR_CAPACITY
    with pytest.raises(sfa.SfaError):
        sfa.offsets_fib(float("nan"))
    with pytest.raises(sfa.SfaError):
        sfa.offsets_fib(-1.0)
    with pytest.raises(sfa.SfaError):
        sfa.stagger_alpha("coprime", 1, 16, 4)
    with pytest.raises(sfa.SfaError):
        sfa.edges_powerlaw(64, 8, 0.8, 30, 8, 0)   # lists exceed the width
    with pytest.raises(sfa.SfaError):
        sfa.rope_table(8, 7, 1e4)


@pytest.mark.parametrize("n,r,sigma,draws,width,seed", [(2048, 8, 0.8, 47, 64, 42), (90, 3, 0.8, 9, 20, 7)])
def test_edges_transpose_bit_exact(n, r, sigma, draws, width, seed):
    edges, count = sfa.edges_powerlaw(n, r, sigma, draws, width, seed)
    inv, inv_count = sfa.edges_transpose(edges, count)
    rinv, rcount = ref_att.transpose_edges(edges, count)
    assert np.array_equal(inv, rinv) and np.array_equal(inv_count, rcount)


def test_edges_transpose_errors():
    lib = sfa.library()
    ip = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    edges = np.array([[1, 2], [0, -1], [0, 1]], dtype=np.int32)
    count = np.array([2, 1, 2], dtype=np.int32)
    inv = np.zeros((3, 1), dtype=np.int32)
    ic = np.zeros(3, dtype=np.int32)
    assert lib.sfa_edges_transpose(3, 2, ip(edges), ip(count), 0, None, None) == 2   # size query
    assert lib.sfa_edges_transpose(3, 2, ip(edges), ip(count), 1, ip(inv), ip(ic)) == sfa.SFA_ERR_CAPACITY
    bad = edges.copy(); bad[1, 0] = 3
    assert lib.sfa_edges_transpose(3, 2, ip(bad), ip(count), 0, None, None) == sfa.SFA_ERR_ARG
    badc = count.copy(); badc[0] = 3
    assert lib.sfa_edges_transpose(3, 2, ip(edges), ip(badc), 0, None, None) == sfa.SFA_ERR_ARG
    assert lib.sfa_edges_transpose(3, 0, ip(edges), ip(count), 0, None, None) == sfa.SFA_ERR_ARG


def test_bwd_edges_validation_and_workspace_size():
    # Every case below is invalid, so no call reaches a device.
    lib = sfa.library()
    a = _prob(batch=2, seqlen=100, hq=4, hkv=4)
    al = lambda e: (e + 63) // 64 * 64
    nb = lib.sfa_bwd_edges_workspace_bytes(ctypes.byref(a), 64)
    # p, dp [B*Hkv][n][width][G]; Dvec / l and 1 / l [B*Hkv][n][G]
    assert nb == (2 * al(2 * 4 * 100 * 64 * 1) + 2 * al(2 * 4 * 100 * 1)) * 4
    assert lib.sfa_bwd_edges_workspace_bytes(ctypes.byref(a), 0) == 0
    t = [FAKE] * 8  # q, k, v, lse, dout, dq, dk, dv
    call = lambda width, invw, ws, wsb, ptrs=t, e=FAKE: lib.sfa_bwd_edges(
        ctypes.byref(a), e, FAKE, width, FAKE, FAKE, invw, *ptrs, ws, wsb, None)
    assert call(0, 8, FAKE, nb) == sfa.SFA_ERR_ARG             # width
    assert call(64, 0, FAKE, nb) == sfa.SFA_ERR_ARG            # inv_width
    assert call(64, 8, FAKE, nb - 4) == sfa.SFA_ERR_CAPACITY   # workspace too small
    assert call(64, 8, MISALIGNED, nb) == sfa.SFA_ERR_CAPACITY
    assert call(64, 8, FAKE, nb, ptrs=[None] + t[1:]) == sfa.SFA_ERR_ARG
    assert call(64, 8, FAKE, nb, ptrs=t[:5] + [MISALIGNED] + t[6:]) == sfa.SFA_ERR_ARG
    assert call(64, 8, FAKE, nb, e=ctypes.c_void_p(0x100002)) == sfa.SFA_ERR_ARG   # edges misaligned


@pytest.mark.parametrize("m,k", [(64, 512), (4, 16), (128, 1024)])
def test_christoffel_signed_bit_exact(m, k):
    assert list(sfa.offsets_christoffel_signed(m, k)) == ref_chr.signed_offsets(m, k)


def test_negative_offsets_need_the_signed_flag():
    lib = sfa.library()
    lo = np.array([-7, 7], dtype=np.int32)
    fr = np.zeros(2, dtype=np.float32)
    a = _prob(lo=lo, frac=fr, window=0)
    assert lib.sfa_bwd_workspace_bytes(ctypes.byref(a)) == 0
    assert _fwd(a) == sfa.SFA_ERR_ARG
    a.flags = sfa.SFA_FLAG_SIGNED_OFFSETS
    assert lib.sfa_bwd_workspace_bytes(ctypes.byref(a)) > 0
    a.flags = 4
    assert lib.sfa_bwd_workspace_bytes(ctypes.byref(a)) == 0


def test_profile_controls_without_launches():
    """The profiling controls work without a device: select one kernel, read
    a kernel that was never launched (zero), select all again, reset."""
    lib = sfa.library()
    assert lib.sfa_profile_select(b"bwd_query") == 0
    assert lib.sfa_profile_select(None) == 0
    sfa.profile_enable(True, only="bwd_query")
    sfa.profile_enable(False)
    sfa.profile_reset()
    assert sfa.profile_read("bwd_query") == (0.0, 0)
    sfa.profile_enable(False, only=None)


def _cpu(shape):
    import torch
    return torch.zeros(shape, dtype=torch.float32)


@pytest.mark.parametrize("which,shape", [
    ("k", (2, 50, 2, 32)),    # k shorter than q's sequence
    ("k", (1, 64, 2, 32)),    # k with fewer batch entries
    ("k", (2, 64, 2, 16)),    # k with another head dim
    ("k", (2, 64, 3, 32)),    # query heads not a multiple of key heads
    ("v", (2, 64, 2, 16)),    # v unlike k
    ("v", (2, 63, 2, 32)),
])
def test_binding_rejects_mismatched_kv_shapes(which, shape):
    # A K or V smaller than Q implies would be read past its end by the
    # kernels (raw pointers); the binding refuses it before any device use.
    q, k, v = _cpu((2, 64, 8, 32)), _cpu((2, 64, 2, 32)), _cpu((2, 64, 2, 32))
    bad = _cpu(shape)
    k_, v_ = (bad, v) if which == "k" else (k, bad)
    lo, fr = sfa.offsets_fib(1.0)
    with pytest.raises(ValueError):
        sfa.fwd(q, k_, v_, 4, lo, fr)
    with pytest.raises(ValueError):
        sfa.bwd(q, k_, v_, _cpu((2, 8, 64)), q, 4, lo, fr)
    e, c = _cpu((64, 8)), _cpu((64,))
    with pytest.raises(ValueError):
        sfa.fwd_edges(q, k_, v_, e, c)
    with pytest.raises(ValueError):
        sfa.bwd_edges(q, k_, v_, _cpu((2, 8, 64)), q, e, c, e, c)


@pytest.mark.parametrize("shape", [(2, 64, 8, 16), (2, 63, 8, 32), (1, 64, 8, 32), (2, 64, 4, 32)])
def test_binding_rejects_mismatched_dout(shape):
    q, k = _cpu((2, 64, 8, 32)), _cpu((2, 64, 2, 32))
    lo, fr = sfa.offsets_fib(1.0)
    with pytest.raises(ValueError):
        sfa.bwd(q, k, k, _cpu((2, 8, 64)), _cpu(shape), 4, lo, fr)
    e, c = _cpu((64, 8)), _cpu((64,))
    with pytest.raises(ValueError):
        sfa.bwd_edges(q, k, k, _cpu((2, 8, 64)), _cpu(shape), e, c, e, c)


def test_binding_rejects_tensors_on_different_devices():
    import torch
    q, k = _cpu((1, 8, 2, 16)), _cpu((1, 8, 1, 16))
    meta = torch.zeros((1, 8, 1, 16), dtype=torch.float32, device="meta")
    lo, fr = sfa.offsets_fib(1.0)
    with pytest.raises(ValueError):
        sfa.fwd(q, k, meta, 0, lo, fr)


def test_noalloc_rejects_oversize_and_invalid_before_any_device_call():
    # The scratch holds SFA_NOALLOC_SCRATCH_BYTES; a larger workspace need is
    # refused with SFA_ERR_CAPACITY, an invalid problem with its own code,
    # both before any HIP call (this runs without a GPU).
    lib = sfa.library()
    lo, frac = sfa.offsets_fib(0.8)
    big = _prob(batch=64, seqlen=1024, lo=lo, frac=frac, window=10)
    assert lib.sfa_bwd_workspace_bytes(ctypes.byref(big)) > sfa.NOALLOC_SCRATCH_BYTES
    base = sfa.base_fib()
    bp = base.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    args = [FAKE] * 9
    rc = lib.sfa_bwd_noalloc(ctypes.byref(big), *args, bp, 0.8, FAKE, None)
    assert rc == sfa.SFA_ERR_CAPACITY
    assert b"static scratch" in lib.sfa_last_error()
    rc = lib.sfa_bwd_noalloc(ctypes.byref(_prob(head_dim=48)), *args, bp, 0.8, FAKE, None)
    assert rc == sfa.SFA_ERR_UNSUPPORTED


def test_absmax_rejects_invalid_before_any_device_call():
    lib = sfa.library()
    res = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails its checks first
    assert lib.sfa_absmax(FAKE, -1, sfa.SFA_BF16, res, None) == sfa.SFA_ERR_ARG
    assert lib.sfa_absmax(FAKE, 16, 7, res, None) == sfa.SFA_ERR_ARG
    assert b"dtype" in lib.sfa_last_error()
    assert lib.sfa_absmax(None, 16, sfa.SFA_F32, res, None) == sfa.SFA_ERR_ARG
    assert lib.sfa_absmax(FAKE, 16, sfa.SFA_F32, None, None) == sfa.SFA_ERR_ARG
    assert lib.sfa_absmax(ctypes.c_void_p(0x100008), 16, sfa.SFA_F32, res, None) == sfa.SFA_ERR_ARG
    assert lib.sfa_absmax(FAKE, 16, sfa.SFA_F32, ctypes.c_void_p(0x100002), None) == sfa.SFA_ERR_ARG
    assert b"aligned" in lib.sfa_last_error()
    # an empty tensor launches nothing
    assert lib.sfa_absmax(None, 0, sfa.SFA_BF16, None, None) == sfa.SFA_OK


def test_range_error_messages_and_limits():
    # SFA_BF16_MAX_ABS is 65504 / sqrt 2 rounded down (a rotated pair stays
    # below f16's largest finite value); SFA_BF16_MIN_ABS is 2^-14
    assert sfa.BF16_MAX_ABS * 2 ** 0.5 <= 65504.0 < (sfa.BF16_MAX_ABS + 1) * 2 ** 0.5
    assert sfa.BF16_MIN_ABS == float(np.finfo(np.float16).tiny)
    assert "overflow" in str(sfa.RangeError("q", 5e4))
    assert "subnormal" in str(sfa.RangeError("dout", 1e-6))
    assert "non-finite" in str(sfa.RangeError("v", float("inf")))
    assert "non-finite" in str(sfa.RangeError("k", float("nan")))
    assert issubclass(sfa.RangeError, ValueError)
