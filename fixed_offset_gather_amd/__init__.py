"""Python binding of libsfa: sparse fixed-offset attention on MI355X.

Argument marshalling only.  Every step of the attention runs in the HIP
kernels of ``libsfa.so`` (built in-tree by ``fixed_offset_gather_amd/build.py``);
the host producers (offsets, schedules, Christoffel offsets, power-law edge
lists, rotary table) run in the same library's C++ code.  PyTorch supplies
device memory and the current stream.  There is no fallback: if the library
is missing, importing this package raises.

Tensor layouts: q, o, dout, dq [B, n, Hq, D]; k, v, dk, dv [B, n, Hkv, D];
lse float32 [B, Hq, n].  dtype float32 or bfloat16, contiguous, on a GPU.
"""

import ctypes
import os

import numpy as np

# torch ships its own HIP runtime with the same soname as the system one.
# Importing torch first makes libsfa bind to that already-loaded runtime, so
# the process holds a single HIP runtime and the library launches on the
# devices and streams torch created.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsfa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libsfa.so is not built; run `python fixed_offset_gather_amd/build.py` "
        "(hipcc, gfx950).  There is no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)

SFA_OK = 0
SFA_ERR_ARG = -1
SFA_ERR_CAPACITY = -2
SFA_ERR_UNSUPPORTED = -3
SFA_ERR_HIP = -4
SFA_F32 = 0
SFA_BF16 = 1
SFA_FLAG_INTERP_KERNEL = 1
SFA_FLAG_SIGNED_OFFSETS = 2
MAX_OFFSETS = 256
MAX_SLOTS = 320
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024
BF16_MAX_ABS = 46318.0
BF16_MIN_ABS = 2.0 ** -14
SCHEDULES = {"fixed": 0, "linear": 1, "coprime": 2}

_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_vp = ctypes.c_void_p


class SfaAttn(ctypes.Structure):
    """Mirror of ``sfa_attn`` in include/sfa.h."""

    _fields_ = [
        ("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
        ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("window", ctypes.c_int32), ("n_off", ctypes.c_int32),
        ("scale", ctypes.c_float), ("flags", ctypes.c_int32),
        ("off_lo", _i32p), ("off_frac", _f32p), ("rope", _vp),
    ]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_c = ctypes
_sig("sfa_last_error", _c.c_char_p, [])
_sig("sfa_version", _c.c_int, [])
_sig("sfa_base_fib", _c.c_int, [_i32p, _c.c_int])
_sig("sfa_base_pow2", _c.c_int, [_i32p, _c.c_int])
_sig("sfa_offsets_scaled", _c.c_int, [_i32p, _c.c_int, _c.c_double, _i32p, _f32p])
_sig("sfa_offsets_fib", _c.c_int, [_c.c_double, _i32p, _f32p, _c.c_int])
_sig("sfa_offsets_pow2", _c.c_int, [_c.c_double, _i32p, _f32p, _c.c_int])
_sig("sfa_stagger_alpha", _c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.POINTER(_c.c_double)])
_sig("sfa_alpha_of_theta", _c.c_int, [_c.c_double, _c.POINTER(_c.c_double), _c.POINTER(_c.c_double)])
_sig("sfa_offsets_christoffel", _c.c_int, [_c.c_int, _c.c_int, _i32p, _c.c_int])
_sig("sfa_offsets_christoffel_signed", _c.c_int, [_c.c_int, _c.c_int, _i32p, _c.c_int])
_sig("sfa_edges_powerlaw", _c.c_int, [_c.c_int, _c.c_int, _c.c_double, _c.c_int, _c.c_int,
                                      _c.c_uint64, _i32p, _i32p])
_sig("sfa_edges_transpose", _c.c_int, [_c.c_int, _c.c_int, _i32p, _i32p, _c.c_int, _i32p, _i32p])
_sig("sfa_rope_table", _c.c_int, [_c.c_int, _c.c_int, _c.c_double, _f32p])
_sig("sfa_fwd", _c.c_int, [_c.POINTER(SfaAttn), _vp, _vp, _vp, _vp, _vp, _vp])
_sig("sfa_fwd_edges", _c.c_int, [_c.POINTER(SfaAttn), _vp, _vp, _c.c_int, _vp, _vp, _vp, _vp, _vp, _vp])
_sig("sfa_bwd_workspace_bytes", _c.c_size_t, [_c.POINTER(SfaAttn)])
_sig("sfa_bwd", _c.c_int, [_c.POINTER(SfaAttn), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           _vp, _i32p, _c.c_double, _vp, _vp, _c.c_size_t, _vp])
_sig("sfa_bwd_noalloc", _c.c_int, [_c.POINTER(SfaAttn), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _i32p, _c.c_double, _vp, _vp])
_sig("sfa_bwd_edges_workspace_bytes", _c.c_size_t, [_c.POINTER(SfaAttn), _c.c_int])
_sig("sfa_bwd_edges", _c.c_int, [_c.POINTER(SfaAttn), _vp, _vp, _c.c_int, _vp, _vp, _c.c_int, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _c.c_size_t, _vp])
_sig("sfa_absmax", _c.c_int, [_vp, _c.c_int64, _c.c_int, _vp, _vp])
_sig("sfa_profile_enable", _c.c_int, [_c.c_int])
_sig("sfa_profile_read", _c.c_int, [_c.c_char_p, _c.POINTER(_c.c_double), _c.POINTER(_c.c_int64)])
_sig("sfa_profile_reset", _c.c_int, [])
_sig("sfa_profile_select", _c.c_int, [_c.c_char_p])


class SfaError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        msg = _lib.sfa_last_error().decode(errors="replace")
        super().__init__("%s failed (%d): %s" % (fn, code, msg))


class RangeError(ValueError):
    """A bfloat16 input outside the range of the kernels' f16 operands."""

    def __init__(self, name, amax):
        self.tensor, self.absmax = name, amax
        if amax != amax or amax == float("inf"):
            why = "holds a non-finite value"
        elif amax > BF16_MAX_ABS:
            why = "has max |x| = %.6g above %.6g (f16 operands would overflow)" % (amax, BF16_MAX_ABS)
        else:
            why = "has max |x| = %.6g below %.6g (f16 operands would be subnormal)" % (amax, BF16_MIN_ABS)
        super().__init__("bfloat16 %s %s" % (name, why))


def _check(fn, rc):
    if rc < 0:
        raise SfaError(fn, rc)
    return rc


def library():
    """The loaded ctypes library (for ABI tests)."""
    return _lib


def _ip(a):
    return a.ctypes.data_as(_i32p)


def _fp(a):
    return a.ctypes.data_as(_f32p)


# ------------------------------------------------------------ host producers

def base_fib():
    out = np.zeros(15, dtype=np.int32)
    _check("sfa_base_fib", _lib.sfa_base_fib(_ip(out), 15))
    return out


def base_pow2():
    out = np.zeros(11, dtype=np.int32)
    _check("sfa_base_pow2", _lib.sfa_base_pow2(_ip(out), 11))
    return out


def offsets_scaled(base, alpha):
    base = np.ascontiguousarray(base, dtype=np.int32)
    lo = np.zeros(len(base), dtype=np.int32)
    frac = np.zeros(len(base), dtype=np.float32)
    _check("sfa_offsets_scaled",
           _lib.sfa_offsets_scaled(_ip(base), len(base), float(alpha), _ip(lo), _fp(frac)))
    return lo, frac


def offsets_fib(alpha):
    lo = np.zeros(15, dtype=np.int32)
    frac = np.zeros(15, dtype=np.float32)
    _check("sfa_offsets_fib", _lib.sfa_offsets_fib(float(alpha), _ip(lo), _fp(frac), 15))
    return lo, frac


def offsets_pow2(alpha):
    lo = np.zeros(11, dtype=np.int32)
    frac = np.zeros(11, dtype=np.float32)
    _check("sfa_offsets_pow2", _lib.sfa_offsets_pow2(float(alpha), _ip(lo), _fp(frac), 11))
    return lo, frac


def stagger_alpha(schedule, layer, L=16, S=7):
    out = ctypes.c_double()
    sched = SCHEDULES[schedule] if isinstance(schedule, str) else int(schedule)
    _check("sfa_stagger_alpha", _lib.sfa_stagger_alpha(sched, layer, L, S, ctypes.byref(out)))
    return out.value


def alpha_of_theta(theta):
    a, d = ctypes.c_double(), ctypes.c_double()
    _check("sfa_alpha_of_theta", _lib.sfa_alpha_of_theta(float(theta), ctypes.byref(a), ctypes.byref(d)))
    return a.value, d.value


def offsets_christoffel(m, k):
    out = np.zeros(max(m, 1), dtype=np.int32)
    cnt = _check("sfa_offsets_christoffel", _lib.sfa_offsets_christoffel(m, k, _ip(out), len(out)))
    return out[:cnt].copy()


def offsets_christoffel_signed(m, k):
    """-O and +O ascending, for a layer run with signed_offsets=True."""
    out = np.zeros(max(2 * m, 1), dtype=np.int32)
    cnt = _check("sfa_offsets_christoffel_signed", _lib.sfa_offsets_christoffel_signed(m, k, _ip(out), len(out)))
    return out[:cnt].copy()


def edges_powerlaw(n, r, sigma, draws, width, seed):
    edges = np.zeros((n, width), dtype=np.int32)
    count = np.zeros(n, dtype=np.int32)
    _check("sfa_edges_powerlaw",
           _lib.sfa_edges_powerlaw(n, r, float(sigma), draws, width, int(seed) & (2**64 - 1),
                                   _ip(edges), _ip(count)))
    return edges, count


def edges_transpose(edges, count):
    """Inverted edge table (host): (inv int32 [n, cap] -1 padded, inv_count int32 [n])."""
    edges = np.ascontiguousarray(edges, dtype=np.int32)
    count = np.ascontiguousarray(count, dtype=np.int32)
    n, width = edges.shape
    cap = _check("sfa_edges_transpose", _lib.sfa_edges_transpose(n, width, _ip(edges), _ip(count), 0, None, None))
    inv = np.zeros((n, cap), dtype=np.int32)
    inv_count = np.zeros(n, dtype=np.int32)
    _check("sfa_edges_transpose",
           _lib.sfa_edges_transpose(n, width, _ip(edges), _ip(count), cap, _ip(inv), _ip(inv_count)))
    return inv, inv_count


def rope_table(n, head_dim, theta):
    """Host float32 [n, head_dim/2, 2] (cos, sin) table built in fp64."""
    out = np.zeros((n, head_dim // 2, 2), dtype=np.float32)
    _check("sfa_rope_table", _lib.sfa_rope_table(n, head_dim, float(theta), _fp(out)))
    return out


# ------------------------------------------------------------ device calls

def _torch():
    import torch
    return torch


def rope_table_device(n, head_dim, theta, device="cuda"):
    """Rotary table copied to the device (None for theta == 0)."""
    if not theta:
        return None
    torch = _torch()
    return torch.from_numpy(rope_table(n, head_dim, theta)).to(device)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return SFA_F32
    if t.dtype == torch.bfloat16:
        return SFA_BF16
    raise TypeError("tensors must be float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _require(t, name, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _check_shapes(q, k, v=None, dout=None):
    """Shapes and devices of the attention tensors, before any other check:
    the C ABI takes raw pointers, so a K, V or dO smaller than Q implies
    would be read (or written) past its end.  q [B, n, Hq, D]; k, v
    [B, n, Hkv, D] with Hq a multiple of Hkv; dout like q."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-d: [B, n, H, D]")
    B, n, hq, d = q.shape
    hkv = k.shape[2]
    if tuple(k.shape) != (B, n, hkv, d):
        raise ValueError("k has shape %s, expected (%d, %d, Hkv, %d)" % (tuple(k.shape), B, n, d))
    if hkv < 1 or hq % hkv:
        raise ValueError("query heads %d are not a multiple of key/value heads %d" % (hq, hkv))
    if v is not None and tuple(v.shape) != tuple(k.shape):
        raise ValueError("v has shape %s, expected %s (like k)" % (tuple(v.shape), tuple(k.shape)))
    if dout is not None and tuple(dout.shape) != tuple(q.shape):
        raise ValueError("dout has shape %s, expected %s (like q)" % (tuple(dout.shape), tuple(q.shape)))
    for t, nm in ((k, "k"), (v, "v"), (dout, "dout")):
        if t is not None and t.device != q.device:
            raise ValueError("%s is on %s, q on %s" % (nm, t.device, q.device))


def absmax(t):
    """Largest |x| of a device tensor (inf or nan if it holds one), from
    sfa_absmax; synchronises the tensor's stream."""
    torch = _torch()
    _require(t, "tensor")
    res = torch.zeros(1, dtype=torch.int32, device=t.device)
    _check("sfa_absmax", _lib.sfa_absmax(_ptr(t), t.numel(), _dtype_code(t), _ptr(res), _stream(t)))
    return float(res.cpu().view(torch.float32).item())


def check_range(**tensors):
    """Raise RangeError for the first bfloat16 tensor outside the kernels'
    f16 operand range: max |x| above BF16_MAX_ABS, non-finite, or nonzero and
    below BF16_MIN_ABS.  float32 tensors are not restricted."""
    torch = _torch()
    for name, t in tensors.items():
        if t is None or t.dtype != torch.bfloat16 or t.numel() == 0:
            continue
        m = absmax(t)
        if not (m <= BF16_MAX_ABS) or 0.0 < m < BF16_MIN_ABS:
            raise RangeError(name, m)


class Problem:
    """Holds an ``sfa_attn`` and the host arrays it points to."""

    def __init__(self, q, k, window=0, lo=None, frac=None, rope=None, scale=0.0, flags=0):
        B, n, hq, d = q.shape
        hkv = k.shape[2]
        self.lo = np.ascontiguousarray(np.zeros(0) if lo is None else lo, dtype=np.int32)
        self.frac = np.ascontiguousarray(np.zeros(0) if frac is None else frac, dtype=np.float32)
        if self.lo.shape != self.frac.shape:
            raise ValueError("lo and frac must have the same length")
        if rope is not None:
            _require(rope, "rope", _torch().float32, (n, d // 2, 2))
        self.rope = rope
        self.c = SfaAttn(B, n, hq, hkv, d, _dtype_code(q), int(window), len(self.lo), float(scale), int(flags),
                         _ip(self.lo), _fp(self.frac), None if rope is None else rope.data_ptr())

    def ref(self):
        return ctypes.byref(self.c)


def fwd(q, k, v, window=0, lo=None, frac=None, rope=None, scale=0.0, want_lse=False, out=None, lse=None,
        interp_kernel=False, signed_offsets=False, range_check=False):
    """Forward over the window 0..window plus shared offsets (lo, frac).

    interp_kernel=True runs the interpolating instantiation even when every
    frac is 0 (SFA_FLAG_INTERP_KERNEL); the result is the same.
    signed_offsets=True admits negative lo (later rows; SFA_FLAG_SIGNED_OFFSETS).
    range_check=True scans bfloat16 inputs first (check_range) and raises
    RangeError, launching nothing, if one is outside the f16 operand range.
    """
    torch = _torch()
    _check_shapes(q, k, v)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, nm, q.dtype)
    if range_check:
        check_range(q=q, k=k, v=v)
    B, n, hq, d = q.shape
    pr = Problem(q, k, window, lo, frac, rope, scale, (SFA_FLAG_INTERP_KERNEL if interp_kernel else 0) |
                 (SFA_FLAG_SIGNED_OFFSETS if signed_offsets else 0))
    o = torch.empty_like(q) if out is None else out
    _require(o, "out", q.dtype, q.shape)
    if want_lse and lse is None:
        lse = torch.empty((B, hq, n), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require(lse, "lse", torch.float32, (B, hq, n))
    _check("sfa_fwd", _lib.sfa_fwd(pr.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(q)))
    return (o, lse) if (want_lse or lse is not None) else o


def fwd_edges(q, k, v, edges, count, rope=None, scale=0.0, want_lse=False, out=None, range_check=False):
    """Forward over per-query edge lists (device int32 [n, width], [n])."""
    torch = _torch()
    _check_shapes(q, k, v)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, nm, q.dtype)
    if range_check:
        check_range(q=q, k=k, v=v)
    B, n, hq, d = q.shape
    _require(edges, "edges", torch.int32)
    _require(count, "count", torch.int32, (n,))
    if edges.dim() != 2 or edges.shape[0] != n:
        raise ValueError("edges must be [n, width]")
    pr = Problem(q, k, 0, None, None, rope, scale)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, hq, n), dtype=torch.float32, device=q.device) if want_lse else None
    _check("sfa_fwd_edges", _lib.sfa_fwd_edges(pr.ref(), _ptr(edges), _ptr(count), int(edges.shape[1]),
                                               _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(q)))
    return (o, lse) if want_lse else o


def bwd_workspace_bytes(q, k, window=0, lo=None, frac=None, rope=None, scale=0.0, signed_offsets=False):
    pr = Problem(q, k, window, lo, frac, rope, scale, SFA_FLAG_SIGNED_OFFSETS if signed_offsets else 0)
    nb = _lib.sfa_bwd_workspace_bytes(pr.ref())
    if nb == 0 and q.numel() > 0:
        raise SfaError("sfa_bwd_workspace_bytes", SFA_ERR_ARG)
    return nb


def bwd(q, k, v, lse, dout, window=0, lo=None, frac=None, rope=None, scale=0.0,
        base=None, alpha=None, workspace=None, want_dd=True, signed_offsets=False, out=None,
        range_check=False):
    """Backward: returns (dq, dk, dv, dd or None, dtheta or None).  out:
    optional (dq, dk, dv) tensors to write (like q, k, v).  range_check as
    for fwd, over q, k, v and dout."""
    torch = _torch()
    _check_shapes(q, k, v, dout)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _require(t, nm, q.dtype)
    if range_check:
        check_range(q=q, k=k, v=v, dout=dout)
    B, n, hq, d = q.shape
    _require(lse, "lse", torch.float32, (B, hq, n))
    pr = Problem(q, k, window, lo, frac, rope, scale, SFA_FLAG_SIGNED_OFFSETS if signed_offsets else 0)
    nb = _lib.sfa_bwd_workspace_bytes(pr.ref())
    if workspace is None:
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        for t, like, nm in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
            _require(t, nm, q.dtype, like.shape)
    nr = len(pr.lo)
    dd = torch.empty(max(nr, 1), dtype=torch.float32, device=q.device) if (want_dd and nr) else None
    dth = None
    base_arr = None
    if base is not None and alpha is not None:
        base_arr = np.ascontiguousarray(base, dtype=np.int32)
        if len(base_arr) != nr:
            raise ValueError("base must have one entry per offset")
        dth = torch.empty(1, dtype=torch.float32, device=q.device)
    _check("sfa_bwd", _lib.sfa_bwd(
        pr.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(dd), None if base_arr is None else _ip(base_arr), float(alpha or 0.0), _ptr(dth),
        _ptr(workspace), workspace.numel(), _stream(q)))
    return dq, dk, dv, dd, dth


def bwd_edges_workspace_bytes(q, k, width, rope=None, scale=0.0):
    pr = Problem(q, k, 0, None, None, rope, scale)
    nb = _lib.sfa_bwd_edges_workspace_bytes(pr.ref(), int(width))
    if nb == 0 and q.numel() > 0:
        raise SfaError("sfa_bwd_edges_workspace_bytes", -1)
    return nb


def bwd_edges(q, k, v, lse, dout, edges, count, inv, inv_count, rope=None, scale=0.0, workspace=None,
              range_check=False):
    """Edge-list backward: returns (dq, dk, dv).  edges/count/inv/inv_count
    are device int32 tensors ([n, width], [n], [n, cap], [n])."""
    torch = _torch()
    _check_shapes(q, k, v, dout)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _require(t, nm, q.dtype)
    if range_check:
        check_range(q=q, k=k, v=v, dout=dout)
    B, n, hq, d = q.shape
    _require(lse, "lse", torch.float32, (B, hq, n))
    for t, nm in ((edges, "edges"), (count, "count"), (inv, "inv"), (inv_count, "inv_count")):
        _require(t, nm, torch.int32)
    if edges.dim() != 2 or edges.shape[0] != n or inv.dim() != 2 or inv.shape[0] != n:
        raise ValueError("edges and inv must be [n, width] and [n, cap]")
    if count.shape != (n,) or inv_count.shape != (n,):
        raise ValueError("count and inv_count must be [n]")
    pr = Problem(q, k, 0, None, None, rope, scale)
    nb = _lib.sfa_bwd_edges_workspace_bytes(pr.ref(), int(edges.shape[1]))
    if workspace is None:
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check("sfa_bwd_edges", _lib.sfa_bwd_edges(
        pr.ref(), _ptr(edges), _ptr(count), int(edges.shape[1]), _ptr(inv), _ptr(inv_count), int(inv.shape[1]),
        _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), workspace.numel(), _stream(q)))
    return dq, dk, dv


# ------------------------------------------------------------ timing

def profile_enable(on=True, only=None):
    """Record HIP events around kernel launches; `only` restricts the
    recording to the launches of that kernel (None: every kernel)."""
    _lib.sfa_profile_select(only.encode() if only else None)
    _lib.sfa_profile_enable(1 if on else 0)


def profile_reset():
    _lib.sfa_profile_reset()


def profile_read(kernel):
    """(total milliseconds, launches) recorded for the named kernel."""
    ms, cnt = ctypes.c_double(), ctypes.c_int64()
    _check("sfa_profile_read", _lib.sfa_profile_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(cnt)))
    return ms.value, cnt.value
