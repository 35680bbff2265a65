"""Kernel timing through the C ABI (sfa_profile_*), on the GPU: every call
records one event pair per timed kernel, taken by the dispatch itself, also
when one call launches a kernel several times (the query pass over more dd
rungs than one launch holds), and a selected kernel is the only one
recorded.  Timing only: the results of these calls are checked elsewhere."""

import numpy as np
import pytest
import torch

import test_gpu_parity as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_off", [12, 100])
def test_profile_records_one_pair_per_call(n_off):
    # 8/2 heads at head dim 64: one query-pass launch holds 64 dd rungs, so
    # 100 Christoffel offsets with the offset gradient take two launches.
    sfa = P._sfa()
    case = P.Case(1, 300, 8, 2, 64, "bf16", seed=5, rope_theta=0.0)
    offs = sfa.offsets_christoffel(n_off, 256)
    assert len(offs) == n_off
    fr = np.zeros(n_off, dtype=np.float32)
    base = offs.astype(np.int32)
    print("profile case: %d offsets" % n_off, flush=True)
    o, lse = sfa.fwd(case.qd, case.kd, case.vd, 0, offs, fr, case.rope, want_lse=True)
    torch.cuda.synchronize()
    try:
        sfa.profile_reset()
        sfa.profile_enable(True)
        for _ in range(3):
            sfa.bwd(case.qd, case.kd, case.vd, lse, case.dod, 0, offs, fr, case.rope, base=base, alpha=1.0)
        torch.cuda.synchronize()
        sfa.profile_enable(False)
        for name in ("bwd_query", "bwd_key"):
            ms, cnt = sfa.profile_read(name)
            print(name, cnt, "launch records, %.4f ms" % ms, flush=True)
            assert cnt == 3 and ms > 0.0, name
        assert sfa.profile_read("fwd_offsets") == (0.0, 0)

        sfa.profile_reset()
        sfa.profile_enable(True, only="bwd_key")
        sfa.fwd(case.qd, case.kd, case.vd, 0, offs, fr, case.rope, want_lse=True)
        sfa.bwd(case.qd, case.kd, case.vd, lse, case.dod, 0, offs, fr, case.rope, base=base, alpha=1.0)
        torch.cuda.synchronize()
        sfa.profile_enable(False)
        ms, cnt = sfa.profile_read("bwd_key")
        assert cnt == 1 and ms > 0.0
        assert sfa.profile_read("bwd_query") == (0.0, 0)
        assert sfa.profile_read("fwd_offsets") == (0.0, 0)
    finally:
        sfa.profile_enable(False, only=None)
        sfa.profile_reset()
