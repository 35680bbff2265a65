"""Index arithmetic of the HIP kernels, checked on the CPU (no GPU).

tests/index_model.py walks each kernel's stages, LDS rows, key-pass ring
slots, rotary rows, workspace offsets and the tiles of the dS bounds the
key pass reads for the slot tables the library
runs: the page-1 learned and fixed layers, the staggered schedule, page 3's
causal and bidirectional Christoffel layers at context 2048, the maximum slot
count, and seeded random tables (interpolated, signed), at full and ragged
lengths.  Two planted mistakes in the model (a rotary row taken from a
negative offset as it stands, a ring slot read without its wrap) must be
caught, so the checks are known to bite.
"""

import numpy as np
import pytest

import index_model as im
from oracle import christoffel as ref_chr
from oracle import offsets as ref_off


def _tables():
    rng = np.random.default_rng(3)
    learned = 0.7886644640192136
    lo_l, fr_l = ref_off.rung_offsets(learned)
    lo_1, fr_1 = ref_off.rung_offsets(1.0)
    causal = np.array(ref_chr.offsets(128, 1024), dtype=np.int64)
    signed = np.concatenate([-causal[::-1], causal])
    rnd_lo = rng.integers(0, 300, size=256)
    rnd_fr = rng.random(256).astype(np.float32)
    rnd_fr[::3] = 0.0
    neg_lo = np.array([-5, -2, 3, -40, 17, 0], dtype=np.int64)
    neg_fr = np.array([0.3, 0.0, 0.6, 0.5, 0.0, 0.25], dtype=np.float32)
    stag = ref_off.schedule_alpha("coprime", 5, 16, 7)
    lo_s, fr_s = ref_off.rung_offsets(stag)
    return {
        "page1_learned": (1024, 10, lo_l, fr_l),
        "page1_fixed": (1024, 8, lo_1, fr_1),
        "page1_staggered_l5": (1024, 12, lo_s, fr_s),
        "christoffel_causal": (2048, 0, causal, np.zeros(128, np.float32)),
        "christoffel_signed": (2048, 0, signed, np.zeros(256, np.float32)),
        "max_slots": (260, 63, rnd_lo, rnd_fr),
        "negative_interpolated": (150, 2, neg_lo, neg_fr),
        "ragged_200": (200, 10, lo_l, fr_l),
        "short_65": (65, 8, lo_l, fr_l),
        "single": (1, 8, lo_l, fr_l),
    }


TABLES = _tables()
IDS = sorted(TABLES)


@pytest.mark.parametrize("name", IDS)
def test_forward_stages_and_rows(name):
    n, W, lo, fr = TABLES[name]
    assert im.forward(n, W, lo, fr, im.BQ_FWD_F32) > 0
    for D, G in ((64, 4), (64, 1), (16, 8)):
        _, bq = im.fwd_h16_shape(D, G)
        assert im.forward(n, W, lo, fr, bq) > 0
    if not np.any(np.asarray(fr) > 0):
        assert im.forward(n, W, lo, fr, im.BQ_FWD_F32, interp=False) > 0


@pytest.mark.parametrize("name", IDS)
def test_query_pass_stages_rows_and_workspace(name):
    n, W, lo, fr = TABLES[name]
    for D, G in ((64, 4), (64, 1), (32, 2), (16, 8)):
        im.query_pass(n, W, lo, fr, D, G, want_dd=True, batch_kv=2)
        im.query_pass(n, W, lo, fr, D, G, want_dd=False)
        im.query_pass(n, W, lo, fr, D, G, want_dd=True, esize=4)


def test_query_pass_rung_windows():
    # 256 rungs at one lane per query head (G = 8, D = 16) take one launch
    # per 16-rung window; at G = 4, D = 64 the 15 Fibonacci rungs take one
    n, W, lo, fr = TABLES["max_slots"]
    assert im.query_pass(n, W, lo, fr, 16, 8) == 16
    n, W, lo, fr = TABLES["page1_learned"]
    assert im.query_pass(n, W, lo, fr, 64, 4) == 1


@pytest.mark.parametrize("name", IDS)
def test_key_pass_ring_holds_each_steps_row(name):
    n, W, lo, fr = TABLES[name]
    for G in (1, 2, 4, 8):
        im.key_pass_h16(n, W, lo, fr, G, batch_kv=2)


@pytest.mark.parametrize("name", IDS)
def test_fp32_key_pass_rows_and_rotary_rows(name):
    n, W, lo, fr = TABLES[name]
    for G in (1, 4):
        im.key_pass_f32(n, W, lo, fr, G)


def test_negative_offset_rotary_row_mistake_is_caught():
    # A future (negative) offset rotated by the table row delta itself reads
    # before the table; the kernel uses row |delta|.
    n, W, lo, fr = TABLES["christoffel_signed"]
    with pytest.raises(im.IndexModelError, match="rotary row"):
        im.key_pass_f32(n, W, lo, fr, 1, rope_row=lambda d: d)
    n, W, lo, fr = TABLES["negative_interpolated"]
    with pytest.raises(im.IndexModelError, match="rotary row"):
        im.key_pass_f32(n, W, lo, fr, 4, rope_row=lambda d: d)


def test_ring_wrap_mistake_is_caught(monkeypatch):
    # The same ring without the wrap at kcap reads past the ring.
    orig = np.where
    n, W, lo, fr = TABLES["page1_learned"]
    kcap = im.key_half_cap(4, 64)

    def no_wrap(cond, a, b):
        if np.isscalar(a) and a == kcap and np.isscalar(b) and b == 0:
            return np.zeros_like(cond, dtype=np.int64)
        return orig(cond, a, b)

    monkeypatch.setattr(im.np, "where", no_wrap)
    with pytest.raises(im.IndexModelError):
        im.key_pass_h16(n, W, lo, fr, 4)


@pytest.mark.parametrize("nseq,nblk", [(64, 32), (32, 64), (16, 2), (8, 1), (3, 32), (64, 7), (5, 3), (1, 1),
                                       (256, 8), (24, 32), (8, 128)])
def test_tile_order_is_a_longest_first_bijection(nseq, nblk):
    # Every workgroup of a launch gets one (sequence, block) in range, each
    # exactly once; canon is the sequence-major numbering of the
    # per-workgroup dd partials; an XCD starts its blocks longest first
    # (the block index never rises along its dispatch order) and, when it
    # holds whole sequences, every block of a sequence runs on one XCD.
    total = nseq * nblk
    ids = np.arange(total)
    seq, blk, canon = im.lpt_seq_block(ids, total, nblk)
    assert seq.min() >= 0 and seq.max() < nseq and blk.min() >= 0 and blk.max() < nblk
    assert len(set(zip(seq.tolist(), blk.tolist()))) == total
    assert np.array_equal(canon, seq * nblk + (nblk - 1 - blk))
    assert np.array_equal(np.sort(canon), ids)
    if total % im.NUM_XCD == 0:
        for x in range(im.NUM_XCD):
            on = ids[ids % im.NUM_XCD == x]  # dispatch order of XCD x
            if (total // im.NUM_XCD) % nblk == 0:
                assert np.all(np.diff(blk[on]) <= 0)
                for s_ in np.unique(seq[on]):
                    assert np.all(seq[ids % im.NUM_XCD != x] != s_)


@pytest.mark.parametrize("halves", [1, 2])
@pytest.mark.parametrize("nseq,nblk,nch", [(64, 8, 4), (8, 16, 4), (32, 16, 4), (3, 5, 4), (16, 8, 4), (2, 1, 4),
                                           (1, 1, 1), (6, 4, 2), (24, 3, 4)])
def test_key_tile_order_is_a_balanced_bijection(halves, nseq, nblk, nch):
    # Each kind of key-pass workgroup covers its T tiles exactly once; with
    # T a multiple of the XCD count every XCD takes T / 8 tiles of each kind
    # (never only the cheaper one), and with whole sequences per XCD its
    # tiles of a kind run longest key block (block 0) first.
    T = nseq * nblk * nch
    ids = np.arange(halves * T)
    part, tile = im.key_tile_order(ids, T, halves, nblk, nch)
    assert part.min() >= 0 and part.max() < halves
    for p_ in range(halves):
        assert np.array_equal(np.sort(tile[part == p_]), np.arange(T))
    if T % im.NUM_XCD == 0:
        xcd = ids % im.NUM_XCD
        for x in range(im.NUM_XCD):
            for p_ in range(halves):
                sel = (xcd == x) & (part == p_)
                assert sel.sum() == T // im.NUM_XCD
                if (T // im.NUM_XCD) % (nblk * nch) == 0:
                    blk = (tile[sel] // nch) % nblk
                    assert np.all(np.diff(blk) >= 0)


def test_step_table_mistake_is_caught(monkeypatch):
    # A step table that gives the farther tap the nearer tap's weight (1 -
    # frac for both) no longer names its slot's taps.
    orig = im.key_step_table

    def wrong_weight_any(sl, n):
        t = orig(sl, n)
        fr = [x[1] for x in sl if x[1] > 0.0]
        out, k = [], 0
        for d, w, first in t:
            if not first:
                w = np.float32(1.0) - np.float32(fr[k])
                k += 1
            out.append((d, w, first))
        return out

    monkeypatch.setattr(im, "key_step_table", wrong_weight_any)
    n, W, lo, fr = TABLES["page1_learned"]
    with pytest.raises(im.IndexModelError, match="step record"):
        im.key_pass_h16(n, W, lo, fr, 4)
