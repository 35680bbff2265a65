"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: max abs error <= 1e-5 for float32 tensors and <= 1e-2 for
bfloat16 tensors (bf16 in, fp32 accumulate, bf16 out).  A bf16 output of
magnitude >= 4 cannot meet 1e-2 on its own rounding (half an ulp is 0.0156
on [4, 8)), so bf16 outputs must lie within 1e-2 plus half a bf16 ulp of
the exact value: the accumulation error, before the final rounding, is what
the 1e-2 bounds.  dd and dtheta are sums over every (query, head) of the
batch (float32 outputs whatever the tensor dtype), so their bound is
relative: |err| <= tol * max(1, |ref|) with the tensor dtype's tol.  Every
check prints its measured errors.  Offsets, edge lists and Christoffel
offsets are produced by the library and were checked bit-exact against the
oracle by the CPU tests.
"""

import numpy as np
import pytest
import torch

import synth_inputs as si
from oracle import attention as ref
from oracle import christoffel as ref_chr
from oracle import offsets as ref_off

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-5, "bf16": 1e-2}


def _sfa():
    import fixed_offset_gather_amd as sfa
    return sfa


def _np(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def _maxerr(a, b):
    return float(np.abs(np.asarray(a, dtype=np.float64) - b).max()) if np.size(b) else 0.0


def _half_ulp_bf16(x):
    """Half the bf16 spacing at |x| (8 significant bits): the error that
    storing an exact value as bf16 can add on its own."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 0.5 * 2.0 ** (np.floor(np.log2(ax)) - 7)


def _excess(gpu, ref, dtype):
    """Max abs error beyond the output's own rounding (bf16: half an ulp of
    the stored value; float32 outputs are compared as they are)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    if not np.size(ref):
        return 0.0
    err = np.abs(gpu - ref)
    if dtype == "bf16":
        err = err - _half_ulp_bf16(np.maximum(np.abs(gpu), np.abs(ref)))
    return float(err.max())


class Case:
    def __init__(self, B, n, hq, hkv, D, dtype, seed=si.SEED, rope_theta=1e4):
        self.B, self.n, self.hq, self.hkv, self.D, self.dtype = B, n, hq, hkv, D, dtype
        self.q, self.k, self.v = si.qkv(B, n, hq, hkv, D, dtype, seed)
        self.do = si.upstream(B, n, hq, D, dtype, seed)
        self.rope_theta = rope_theta
        self.rope = _sfa().rope_table_device(n, D, rope_theta, DEV)
        self.qd, self.kd, self.vd, self.dod = (t.to(DEV) for t in (self.q, self.k, self.v, self.do))

    def f64(self, sel=slice(None)):
        return [si.to_f64(t[sel]) for t in (self.q, self.k, self.v, self.do)]


def _fwd_check(case, W, lo, frac, sel=slice(None), tol=None, signed=False):
    sfa = _sfa()
    o, lse = sfa.fwd(case.qd, case.kd, case.vd, W, lo, frac, case.rope, want_lse=True, signed_offsets=signed)
    torch.cuda.synchronize()
    q, k, v, _ = case.f64(sel)
    ro, rl = ref.forward(q, k, v, W, lo, frac, case.rope_theta)
    tol = tol or TOL[case.dtype]
    eo = _excess(_np(o)[sel], ro, case.dtype)
    el = _maxerr(_np(lse)[sel], rl)
    print("fwd max err o=%.3g (raw %.3g) lse=%.3g" % (eo, _maxerr(_np(o)[sel], ro), el), flush=True)
    assert eo <= tol and el <= tol
    return o, lse


def _bwd_check(case, W, lo, frac, alpha, base, sel=slice(None), tol=None, grad_tol=None, want_dd=True,
               signed=False):
    sfa = _sfa()
    o, lse = sfa.fwd(case.qd, case.kd, case.vd, W, lo, frac, case.rope, want_lse=True, signed_offsets=signed)
    dq, dk, dv, dd, dth = sfa.bwd(case.qd, case.kd, case.vd, lse, case.dod, W, lo, frac, case.rope,
                                  base=base if want_dd else None, alpha=alpha if want_dd else None,
                                  want_dd=want_dd, signed_offsets=signed)
    if not want_dd:
        assert dd is None and dth is None
    torch.cuda.synchronize()
    g = ref.backward(*case.f64(sel), W, lo, frac, case.rope_theta)
    tol = tol or TOL[case.dtype]
    grad_tol = grad_tol or tol
    errs = {nm: _excess(_np(t)[sel], g[nm], case.dtype) for nm, t in (("dq", dq), ("dk", dk), ("dv", dv))}
    raw = {nm: _maxerr(_np(t)[sel], g[nm]) for nm, t in (("dq", dq), ("dk", dk), ("dv", dv))}
    print("bwd max err beyond output rounding", {k_: "%.3g" % e for k_, e in errs.items()},
          "raw", {k_: "%.3g" % e for k_, e in raw.items()}, flush=True)
    for nm, e in errs.items():
        assert e <= tol, nm
    if want_dd and sel == slice(None) and len(lo):
        rdd = g["dd"]
        rth = ref.dtheta_from_dd(rdd, base, alpha)
        bdd = grad_tol * np.maximum(1.0, np.abs(rdd))
        bth = grad_tol * max(1.0, abs(rth))
        add = np.abs(_np(dd) - rdd)
        ath = abs(float(dth.item()) - rth)
        print("dd rel err (|err| / max(1,|ref|)) per rung:",
              " ".join("%.2g" % x for x in add / np.maximum(1.0, np.abs(rdd))), flush=True)
        print("dd worst err/bound %.3g (rung %d, ref %.6g)  dtheta abs err %.3g bound %.3g (ref %.8g)"
              % (float((add / bdd).max()), int((add / bdd).argmax()), float(rdd[int((add / bdd).argmax())]),
                 ath, bth, rth), flush=True)
        assert np.all(add <= bdd) and ath <= bth
    return dq, dk, dv, dd, dth


# ---------------------------------------------------------------- small cases

def test_tiny_fp32_forward():
    case = Case(1, 64, 1, 1, 16, "f32")
    lo, frac = _sfa().offsets_fib(0.75)
    _fwd_check(case, 4, lo, frac)


def test_tiny_fp32_backward():
    case = Case(1, 64, 1, 1, 16, "f32")
    lo, frac = _sfa().offsets_fib(0.75)
    _bwd_check(case, 4, lo, frac, 0.75, _sfa().base_fib())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hq,hkv,D", [(8, 2, 64), (4, 4, 64), (8, 1, 32), (2, 1, 16), (8, 1, 16)])
@pytest.mark.parametrize("W,alpha", [(8, 1.0), (3, 0.713), (0, 1.37)])
def test_forward_multi_tile_ragged(dtype, hq, hkv, D, W, alpha):
    case = Case(2, 200, hq, hkv, D, dtype, seed=7)
    lo, frac = _sfa().offsets_fib(alpha)
    _fwd_check(case, W, lo, frac)


@pytest.mark.parametrize("hq,hkv,D", [(4, 2, 64), (16, 2, 64), (8, 2, 32), (8, 1, 32)])
def test_backward_packed_key_rows_group_shapes(hq, hkv, D):
    # bf16 with two or more heads per KV head: the query pass writes the key
    # pass's rows packed as f16 head pairs (8, 4 and 2 dims per lane, 1 to 4
    # head pairs), which the key pass stages by copying
    case = Case(2, 150, hq, hkv, D, "bf16", seed=37, rope_theta=1e4)
    lo, frac = _sfa().offsets_fib(0.83)
    _bwd_check(case, 6, lo, frac, 0.83, _sfa().base_fib())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hq,hkv,D", [(8, 2, 64), (4, 4, 64), (2, 1, 32), (8, 1, 16)])
@pytest.mark.parametrize("W,alpha", [(10, 0.713), (2, 1.0)])
def test_backward_multi_tile_ragged(dtype, hq, hkv, D, W, alpha):
    case = Case(2, 200, hq, hkv, D, dtype, seed=11)
    lo, frac = _sfa().offsets_fib(alpha)
    _bwd_check(case, W, lo, frac, alpha, _sfa().base_fib())


def test_forward_without_rope_and_pow2_base():
    case = Case(2, 130, 8, 2, 64, "f32", seed=3, rope_theta=0.0)
    lo, frac = _sfa().offsets_pow2(0.9)
    _fwd_check(case, 6, lo, frac)


def test_integer_offsets_equal_window_slots_bitwise():
    # An offset with frac == 0 at distance d is the plain integer gather of row
    # i - d; listing distances 1..3 as offsets or as window slots must give
    # bit-identical outputs (the slots are processed in the same order).
    sfa = _sfa()
    case = Case(2, 150, 8, 2, 64, "bf16", seed=5)
    lo = np.array([1, 2, 3], dtype=np.int32)
    fr = np.zeros(3, dtype=np.float32)
    o1, l1 = sfa.fwd(case.qd, case.kd, case.vd, 0, lo, fr, case.rope, want_lse=True)
    o2, l2 = sfa.fwd(case.qd, case.kd, case.vd, 3, None, None, case.rope, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W,base", [(8, "fib"), (0, "fib"), (8, "pow2")])
def test_integer_instantiation_bitwise_equals_interpolating_kernel(dtype, W, base):
    # alpha = 1: every rung is an integer distance, so the library runs the
    # integer instantiation (no interpolation code); the interpolating
    # instantiation forced on the same layer must give the same bits.
    sfa = _sfa()
    case = Case(4, 1024, 8, 2, 64, dtype, seed=13)
    lo, fr = (sfa.offsets_fib if base == "fib" else sfa.offsets_pow2)(1.0)
    assert not fr.any()
    o1, l1 = sfa.fwd(case.qd, case.kd, case.vd, W, lo, fr, case.rope, want_lse=True)
    o2, l2 = sfa.fwd(case.qd, case.kd, case.vd, W, lo, fr, case.rope, want_lse=True, interp_kernel=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    _fwd_check(case, W, lo, fr, sel=slice(0, 1))


def test_integer_alpha_interpolation_path_bitwise():
    # alpha = 1: every rung has frac = 0; the same rungs given as exact
    # integer distances (frac = 0 written explicitly) are bit-identical, and
    # a frac of 0 through the lerp equals the plain gather.
    sfa = _sfa()
    case = Case(1, 1024, 8, 2, 64, "bf16", seed=9)
    lo, fr = sfa.offsets_fib(1.0)
    assert not fr.any()
    o1 = sfa.fwd(case.qd, case.kd, case.vd, 8, lo, fr, case.rope)
    o2 = sfa.fwd(case.qd, case.kd, case.vd, 8, np.array(ref_off.FIB_BASE, dtype=np.int32),
                 np.zeros(15, dtype=np.float32), case.rope)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_christoffel_small_and_reduced_pair():
    sfa = _sfa()
    case = Case(2, 300, 4, 4, 64, "bf16", seed=13, rope_theta=0.0)
    offs = sfa.offsets_christoffel(3, 8)
    assert list(offs) == ref_chr.offsets(3, 8)
    _fwd_check(case, 0, offs, np.zeros(len(offs), dtype=np.float32))


def test_edge_lists_small():
    sfa = _sfa()
    case = Case(2, 300, 4, 4, 64, "bf16", seed=17, rope_theta=0.0)
    e, c = sfa.edges_powerlaw(300, 4, 0.8, 20, 32, 42)
    o, lse = sfa.fwd_edges(case.qd, case.kd, case.vd, torch.from_numpy(e).to(DEV),
                           torch.from_numpy(c).to(DEV), want_lse=True)
    torch.cuda.synchronize()
    q, k, v, _ = case.f64()
    ro, rl = ref.forward_edges(q, k, v, e, c)
    assert _excess(_np(o), ro, "bf16") <= 1e-2 and _maxerr(_np(lse), rl) <= 1e-2


def test_edge_lists_with_rope_fp32():
    sfa = _sfa()
    case = Case(1, 100, 2, 1, 32, "f32", seed=19, rope_theta=1e4)
    e, c = sfa.edges_powerlaw(100, 2, 0.8, 10, 16, 3)
    o = sfa.fwd_edges(case.qd, case.kd, case.vd, torch.from_numpy(e).to(DEV), torch.from_numpy(c).to(DEV),
                      rope=case.rope)
    torch.cuda.synchronize()
    q, k, v, _ = case.f64()
    ro, _ = ref.forward_edges(q, k, v, e, c, 1e4)
    assert _maxerr(_np(o), ro) <= 1e-5


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("n", [1, 2, 5, 63, 64, 65])
def test_short_sequences(n):
    case = Case(3, n, 8, 2, 64, "f32", seed=23)
    lo, frac = _sfa().offsets_fib(0.713)
    _fwd_check(case, 8, lo, frac)
    _bwd_check(case, 8, lo, frac, 0.713, _sfa().base_fib())


def test_self_only_returns_values():
    sfa = _sfa()
    case = Case(1, 77, 4, 2, 32, "f32", seed=29)
    o = sfa.fwd(case.qd, case.kd, case.vd, 0, None, None, case.rope)
    torch.cuda.synchronize()
    want = case.v.repeat_interleave(2, dim=2)
    assert torch.equal(o.cpu(), want)


def test_offsets_beyond_sequence_are_masked():
    case = Case(1, 100, 8, 2, 64, "f32", seed=31)
    lo = np.array([150, 400, 99, 100], dtype=np.int32)
    fr = np.array([0.0, 0.5, 0.25, 0.0], dtype=np.float32)
    _fwd_check(case, 2, lo, fr)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_maximum_slot_count(dtype):
    # The full table: 320 slots, the maximum 256 offsets (a third of them
    # integer) plus a window of 63, with 4 query heads per KV head: the
    # forward's LDS copy of the table, the key pass's five 64-slot columns,
    # and dd of 256 rungs in the query pass, four launches of a 64-rung
    # window each.
    sfa = _sfa()
    rng = np.random.default_rng(0)
    lo = rng.integers(0, 300, size=sfa.MAX_OFFSETS).astype(np.int32)
    fr = rng.random(sfa.MAX_OFFSETS).astype(np.float32)
    fr[::3] = 0.0
    case = Case(1, 260, 8, 2, 64, dtype, seed=37)
    W = sfa.MAX_SLOTS - 1 - sfa.MAX_OFFSETS
    _fwd_check(case, W, lo, fr)
    _bwd_check(case, W, lo, fr, 1.0, np.ones(sfa.MAX_OFFSETS, dtype=np.int32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_maximum_window(dtype):
    # 320 slots as a window of 191 and 128 offsets: stages of up to 128 rows
    # hold many window slots, and two 64-rung dd windows.
    sfa = _sfa()
    rng = np.random.default_rng(1)
    lo = rng.integers(0, 300, size=128).astype(np.int32)
    fr = rng.random(128).astype(np.float32)
    fr[::3] = 0.0
    case = Case(1, 260, 8, 2, 64, dtype, seed=38)
    W = sfa.MAX_SLOTS - 1 - 128
    _fwd_check(case, W, lo, fr)
    _bwd_check(case, W, lo, fr, 1.0, np.ones(128, dtype=np.int32))


def test_backward_guard_bands_untouched():
    # dQ, dK, dV and the workspace placed inside sentinel-filled buffers:
    # nothing outside them is written, and the results still match.
    sfa = _sfa()
    case = Case(2, 200, 8, 2, 64, "bf16", seed=47)
    lo, fr = sfa.offsets_fib(0.713)
    o, lse = sfa.fwd(case.qd, case.kd, case.vd, 10, lo, fr, case.rope, want_lse=True)
    pad = 4096

    def guarded(like):
        buf = torch.full((like.numel() + 2 * pad,), 12345.0, dtype=like.dtype, device=DEV)
        return buf, buf[pad:pad + like.numel()].view(like.shape)

    (bq, dq), (bk, dk), (bv, dv) = guarded(case.qd), guarded(case.kd), guarded(case.vd)
    nb = sfa.bwd_workspace_bytes(case.qd, case.kd, 10, lo, fr, case.rope)
    wbuf = torch.full((nb + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = wbuf[pad:pad + nb]
    _, _, _, dd, dth = sfa.bwd(case.qd, case.kd, case.vd, lse, case.dod, 10, lo, fr, case.rope,
                               base=sfa.base_fib(), alpha=0.713, workspace=ws, out=(dq, dk, dv))
    torch.cuda.synchronize()
    for buf in (bq, bk, bv):
        assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[-pad:] == 12345.0)
    assert torch.all(wbuf[:pad] == 0xA5) and torch.all(wbuf[-pad:] == 0xA5)
    g = ref.backward(*case.f64(), 10, lo, fr, 1e4)
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert _excess(_np(t), g[nm], "bf16") <= 1e-2, nm
    assert np.all(np.abs(_np(dd) - g["dd"]) <= 1e-2 * np.maximum(1.0, np.abs(g["dd"])))


def test_empty_batch():
    sfa = _sfa()
    q = torch.empty((0, 64, 8, 64), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((0, 64, 2, 64), dtype=torch.bfloat16, device=DEV)
    lo, fr = sfa.offsets_fib(1.0)
    o, lse = sfa.fwd(q, k, k, 8, lo, fr, None, want_lse=True)
    dq, dk, dv, dd, dth = sfa.bwd(q, k, k, lse, q, 8, lo, fr, None, base=sfa.base_fib(), alpha=1.0)
    torch.cuda.synchronize()
    assert o.shape == q.shape and float(dd.abs().sum()) == 0.0 and float(dth.item()) == 0.0


def test_backward_is_deterministic():
    sfa = _sfa()
    case = Case(2, 300, 8, 2, 64, "bf16", seed=41)
    lo, fr = sfa.offsets_fib(0.713)
    o, lse = sfa.fwd(case.qd, case.kd, case.vd, 10, lo, fr, case.rope, want_lse=True)
    r1 = sfa.bwd(case.qd, case.kd, case.vd, lse, case.dod, 10, lo, fr, case.rope, base=sfa.base_fib(),
                 alpha=0.713)
    r2 = sfa.bwd(case.qd, case.kd, case.vd, lse, case.dod, 10, lo, fr, case.rope, base=sfa.base_fib(),
                 alpha=0.713)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_output_guard_bands_untouched():
    sfa = _sfa()
    case = Case(2, 200, 8, 2, 64, "bf16", seed=43)
    lo, fr = sfa.offsets_fib(0.713)
    numel = case.q.numel()
    pad = 4096
    buf = torch.full((numel + 2 * pad,), 12345.0, dtype=torch.bfloat16, device=DEV)
    out = buf[pad:pad + numel].view(case.q.shape)
    sfa.fwd(case.qd, case.kd, case.vd, 10, lo, fr, case.rope, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[pad + numel:] == 12345.0)
    q, k, v, _ = case.f64()
    ro, _ = ref.forward(q, k, v, 10, lo, fr, 1e4)
    assert _excess(_np(out), ro, "bf16") <= 1e-2


# ------------------------------------------------------- full-size workloads

def test_page1_fixed_full_size():
    w = si.WORKLOADS["page1_fixed"]
    case = Case(w["batch"], w["seqlen"], w["hq"], w["hkv"], w["head_dim"], w["dtype"])
    lo, frac = _sfa().offsets_fib(w["alpha"])
    _fwd_check(case, w["window"], lo, frac)


def test_page1_staggered_all_layers_full_size():
    sfa = _sfa()
    w = si.WORKLOADS["page1_staggered"]
    case = Case(w["batch"], w["seqlen"], w["hq"], w["hkv"], w["head_dim"], w["dtype"])
    calls = []
    for W in w["windows"]:
        for layer in range(w["layers"]):
            calls.append((W, "fib", sfa.stagger_alpha("coprime", layer, w["layers"], w["stride"])))
    for layer in range(w["layers"]):
        calls.append((8, "pow2", sfa.stagger_alpha("coprime", layer, w["layers"], w["stride"])))
    calls.append((8, "pow2", 1.0))
    assert len(calls) == 81
    for idx, (W, basis, alpha) in enumerate(calls):
        lo, frac = (sfa.offsets_fib if basis == "fib" else sfa.offsets_pow2)(alpha)
        b = idx % case.B
        print("call %d W=%d %s alpha=%.6f sampled sequence %d" % (idx, W, basis, alpha, b), flush=True)
        _fwd_check(case, W, lo, frac, sel=slice(b, b + 1))


def test_page1_learned_step_full_size():
    sfa = _sfa()
    w = si.WORKLOADS["page1_learned_step"]
    case = Case(w["batch"], w["seqlen"], w["hq"], w["hkv"], w["head_dim"], w["dtype"])
    alpha = si.learned_alpha()
    lo, frac = sfa.offsets_fib(alpha)
    print("alpha", alpha, flush=True)
    _bwd_check(case, w["window"], lo, frac, alpha, sfa.base_fib())


@pytest.mark.parametrize("n", [2048, 4096, 8192])
@pytest.mark.parametrize("alpha", [1.0, 0.7886])
def test_length_extrapolation_forward(n, alpha):
    # The page-1 layer at longer contexts with unchanged offsets: 32,768
    # tokens per batch as 32768 / n sequences; sequence 0 compared in full.
    sfa = _sfa()
    case = Case(32768 // n, n, 8, 2, 64, "bf16", seed=21)
    lo, frac = sfa.offsets_fib(alpha)
    _fwd_check(case, 8, lo, frac, sel=slice(0, 1))


def test_length_extrapolation_backward_4096():
    sfa = _sfa()
    case = Case(2, 4096, 8, 2, 64, "bf16", seed=22)
    alpha = 0.7886
    lo, frac = sfa.offsets_fib(alpha)
    _bwd_check(case, 10, lo, frac, alpha, sfa.base_fib())


def test_christoffel_backward_full_size():
    # Page 3's layer trained: self + 128 carry-word offsets (129 slots, the
    # general slot-table path of the key pass), no rotation, no offset
    # gradient requested; sequence 0 of 8 compared.
    sfa = _sfa()
    w = si.WORKLOADS["ctx2048_christoffel"]
    case = Case(w["batch"], w["seqlen"], w["hq"], w["hkv"], w["head_dim"], w["dtype"], rope_theta=0.0)
    offs = sfa.offsets_christoffel(w["m"], w["k"])
    _bwd_check(case, 0, offs, np.zeros(len(offs), dtype=np.float32), None, None, sel=slice(0, 1), want_dd=False)


def test_christoffel_backward_full_size_with_dd():
    # Page 3's causal layer (self + 128 carry-word offsets, context 2048, 8
    # sequences, one query head per KV head) with the offset gradient: every
    # rung is an integer distance, dd_k is the derivative toward the farther
    # row; all 8 sequences compared, dd summed over the whole batch.
    sfa = _sfa()
    w = si.WORKLOADS["ctx2048_christoffel"]
    case = Case(w["batch"], w["seqlen"], w["hq"], w["hkv"], w["head_dim"], w["dtype"], rope_theta=0.0)
    offs = sfa.offsets_christoffel(w["m"], w["k"])
    fr = np.zeros(len(offs), dtype=np.float32)
    _bwd_check(case, 0, offs, fr, 1.0, offs.astype(np.int32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_without_dd_integer_rungs(dtype):
    # alpha = 1 without dd: integer rungs skip their weight-0 second tap.
    sfa = _sfa()
    case = Case(2, 200, 8, 2, 64, dtype, seed=17)
    lo, frac = sfa.offsets_fib(1.0)
    _bwd_check(case, 8, lo, frac, None, None, want_dd=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_more_than_64_slots_with_dd(dtype):
    # 97 slots (self + 96 carry-word offsets): the key pass reads its slot
    # table from three VGPR columns; dd and dtheta over the integer offsets.
    sfa = _sfa()
    case = Case(2, 300, 4, 4, 32, dtype, seed=19, rope_theta=0.0)
    offs = sfa.offsets_christoffel(96, 256)
    assert len(offs) == 96
    fr = np.zeros(len(offs), dtype=np.float32)
    _bwd_check(case, 0, offs, fr, 1.0, offs.astype(np.int32))


def _edge_bwd_check(case, edges, count, sel=slice(None), tol=None):
    sfa = _sfa()
    ed, cd = torch.from_numpy(edges).to(DEV), torch.from_numpy(count).to(DEV)
    inv, ic = sfa.edges_transpose(edges, count)
    invd, icd = torch.from_numpy(inv).to(DEV), torch.from_numpy(ic).to(DEV)
    o, lse = sfa.fwd_edges(case.qd, case.kd, case.vd, ed, cd, case.rope, want_lse=True)
    dq, dk, dv = sfa.bwd_edges(case.qd, case.kd, case.vd, lse, case.dod, ed, cd, invd, icd, case.rope)
    torch.cuda.synchronize()
    g = ref.backward_edges(*case.f64(sel), edges, count, case.rope_theta)
    tol = tol or TOL[case.dtype]
    errs = {nm: _excess(_np(t)[sel], g[nm], case.dtype) for nm, t in (("dq", dq), ("dk", dk), ("dv", dv))}
    print("edge bwd max err beyond output rounding", {k_: "%.3g" % e for k_, e in errs.items()}, flush=True)
    for nm, e in errs.items():
        assert e <= tol, nm
    return dq, dk, dv


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hq,hkv,D", [(8, 2, 64), (4, 4, 64), (2, 1, 32), (8, 1, 16)])
@pytest.mark.parametrize("theta", [1e4, 0.0])
def test_edge_backward_multi_tile_ragged(dtype, hq, hkv, D, theta):
    sfa = _sfa()
    case = Case(2, 200, hq, hkv, D, dtype, seed=23, rope_theta=theta)
    edges, count = sfa.edges_powerlaw(200, 3, 0.8, 12, 24, 11)
    _edge_bwd_check(case, edges, count)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("width,radius,draws", [(13, 2, 6), (7, 1, 3)])
def test_edge_lists_width_not_a_multiple_of_the_chunk(dtype, width, radius, draws):
    # The forward reads its lists in chunks of 4 entries; a width that is not
    # a multiple of 4 ends the last chunk past the list (the index is clamped
    # there) and the last query's list ends the buffer.
    sfa = _sfa()
    case = Case(2, 150, 8, 2, 64, dtype, seed=29, rope_theta=1e4)
    edges, count = sfa.edges_powerlaw(150, radius, 0.8, draws, width, 5)
    assert edges.shape == (150, width) and int(count.max()) <= width
    o = sfa.fwd_edges(case.qd, case.kd, case.vd, torch.from_numpy(edges).to(DEV),
                      torch.from_numpy(count).to(DEV), rope=case.rope)
    torch.cuda.synchronize()
    q, k, v, _ = case.f64()
    ro, _ = ref.forward_edges(q, k, v, edges, count, 1e4)
    if dtype == "bf16":
        assert _excess(_np(o), ro, "bf16") <= 1e-2
    else:
        assert _maxerr(_np(o), ro) <= 1e-5
    _edge_bwd_check(case, edges, count)


def test_edge_backward_ctx2048_powerlaw_full_size_and_deterministic():
    sfa = _sfa()
    w = si.WORKLOADS["ctx2048_powerlaw"]
    case = Case(w["batch"], w["seqlen"], w["hq"], w["hkv"], w["head_dim"], w["dtype"], rope_theta=0.0)
    edges, count = sfa.edges_powerlaw(w["seqlen"], w["radius"], w["sigma"], w["draws"], w["width"], si.SEED)
    a = _edge_bwd_check(case, edges, count, sel=slice(0, 1))
    b = _edge_bwd_check(case, edges, count, sel=slice(0, 1))
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [0, 3])
def test_signed_christoffel_multi_tile(dtype, W):
    # Page 3's bidirectional layer by signed offsets: keys i - o and i + o.
    sfa = _sfa()
    case = Case(2, 200, 8, 2, 64, dtype, seed=29)
    offs = sfa.offsets_christoffel_signed(8, 64)
    assert offs[0] == -63 and offs[-1] == 63
    fr = np.zeros(len(offs), dtype=np.float32)
    _fwd_check(case, W, offs, fr, signed=True)
    _bwd_check(case, W, offs, fr, 1.0, np.abs(offs).astype(np.int32), signed=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_negative_interpolated_offsets(dtype):
    # Later rows between i + 4 and i + 5 (weight 0.3 on i + 4), an integer
    # future offset, and an ordinary rung, with dd.
    sfa = _sfa()
    case = Case(2, 150, 4, 2, 32, dtype, seed=31)
    lo = np.array([-5, -2, 3], dtype=np.int32)
    fr = np.array([0.3, 0.0, 0.6], dtype=np.float32)
    _bwd_check(case, 2, lo, fr, 1.0, np.array([5, 2, 3], dtype=np.int32), signed=True)


@pytest.mark.parametrize("m,k", [(128, 1024), (64, 512)])
def test_bidirectional_christoffel_full_size(m, k):
    # Page 3's example m = 128, k = 1024 made bidirectional: 256 signed
    # offsets + self = 257 slots (more than five 64-slot columns of the key
    # pass's slot table); and m = 64, k = 512 (129 slots).  Context 2048,
    # sequence 0 of 8.
    sfa = _sfa()
    w = si.WORKLOADS["ctx2048_christoffel"]
    case = Case(w["batch"], w["seqlen"], w["hq"], w["hkv"], w["head_dim"], w["dtype"], rope_theta=0.0)
    offs = sfa.offsets_christoffel_signed(m, k)
    assert len(offs) == 2 * m
    fr = np.zeros(len(offs), dtype=np.float32)
    _fwd_check(case, 0, offs, fr, sel=slice(0, 1), signed=True)
    _bwd_check(case, 0, offs, fr, None, None, sel=slice(0, 1), want_dd=False, signed=True)


def test_ctx2048_christoffel_full_size():
    sfa = _sfa()
    w = si.WORKLOADS["ctx2048_christoffel"]
    case = Case(w["batch"], w["seqlen"], w["hq"], w["hkv"], w["head_dim"], w["dtype"], rope_theta=0.0)
    offs = sfa.offsets_christoffel(w["m"], w["k"])
    assert len(offs) == 128 and list(offs[:3]) == [7, 15, 23]
    _fwd_check(case, 0, offs, np.zeros(len(offs), dtype=np.float32), sel=slice(0, 2))


def test_ctx2048_powerlaw_full_size():
    sfa = _sfa()
    w = si.WORKLOADS["ctx2048_powerlaw"]
    case = Case(w["batch"], w["seqlen"], w["hq"], w["hkv"], w["head_dim"], w["dtype"], rope_theta=0.0)
    e, c = sfa.edges_powerlaw(w["seqlen"], w["radius"], w["sigma"], w["draws"], w["width"], si.SEED)
    o, lse = sfa.fwd_edges(case.qd, case.kd, case.vd, torch.from_numpy(e).to(DEV),
                           torch.from_numpy(c).to(DEV), want_lse=True)
    torch.cuda.synchronize()
    q, k, v, _ = case.f64(slice(0, 2))
    ro, rl = ref.forward_edges(q, k, v, e, c)
    assert _excess(_np(o)[:2], ro, "bf16") <= 1e-2 and _maxerr(_np(lse)[:2], rl) <= 1e-2
