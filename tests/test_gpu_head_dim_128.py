"""Head dim 128 (bf16 tensors; fp32 ones are refused there), on the GPU
through the C ABI against the oracle at the bf16 bounds: the shared-offset
forward and backward (interpolated rungs, RoPE, the offset gradient) for one,
two, four and eight heads per KV head over ragged multi-tile sequences, the
Christoffel layer with signed offsets, and power-law edge lists."""

import numpy as np
import pytest

import test_gpu_parity as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (4, 2), (8, 1), (16, 2)])
@pytest.mark.parametrize("W,alpha", [(10, 0.713), (3, 1.0)])
def test_forward_head_dim_128(hq, hkv, W, alpha):
    case = P.Case(2, 150, hq, hkv, 128, "bf16", seed=41, rope_theta=1e4)
    lo, frac = P._sfa().offsets_fib(alpha)
    P._fwd_check(case, W, lo, frac)


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (4, 2), (8, 1), (16, 2)])
def test_backward_head_dim_128(hq, hkv):
    case = P.Case(2, 150, hq, hkv, 128, "bf16", seed=43, rope_theta=1e4)
    lo, frac = P._sfa().offsets_fib(0.79)
    P._bwd_check(case, 8, lo, frac, 0.79, P._sfa().base_fib())


def test_signed_christoffel_head_dim_128():
    sfa = P._sfa()
    case = P.Case(1, 180, 4, 4, 128, "bf16", seed=47)
    lo = sfa.offsets_christoffel_signed(8, 48)
    fr = np.zeros(len(lo), np.float32)
    P._fwd_check(case, 2, lo, fr, signed=True)
    P._bwd_check(case, 2, lo, fr, 1.0, np.abs(lo).astype(np.int32), want_dd=False, signed=True)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (16, 2)])
@pytest.mark.parametrize("theta", [1e4, 0.0])
def test_edge_lists_head_dim_128(hq, hkv, theta):
    sfa = P._sfa()
    case = P.Case(2, 160, hq, hkv, 128, "bf16", seed=53, rope_theta=theta)
    edges, count = sfa.edges_powerlaw(160, 3, 0.8, 12, 24, 17)
    P._edge_bwd_check(case, edges, count)
