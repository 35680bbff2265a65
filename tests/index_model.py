"""Host model of the index arithmetic of the HIP kernels (test infrastructure).

Each function below walks one kernel of fixed_offset_gather_amd/csrc the way
the kernel walks its work: the slot-table order and stage grouping, the LDS
rows a stage stages and the rows each lane then reads, the LDS ring of the
bf16 key pass (which slot holds which query row), the rotary-table rows and
the workspace offsets.  Lanes are numpy vectors, one element per thread, so a
whole workgroup is checked at once.  Every address is checked against the
buffer it indexes (raising IndexModelError), and ring reads are checked to
find the row they expect.  The model follows the kernels' source: a change to
their index arithmetic must be made here too (the kernel functions are named
in each docstring).  It computes nothing of the attention itself.
"""

import numpy as np

MAX_SLOTS = 320
BQ_FWD_F32 = 64      # sfa_fwd.hip: BQ
CAP = 128            # sfa_fwd.hip / sfa_bwd.hip: kCap
KB_H16 = 256         # sfa_bwd.hip: kKeyBlockH16


class IndexModelError(AssertionError):
    pass


def check(cond, what):
    if not np.all(cond):
        raise IndexModelError(what)


# ------------------------------------------------------------ tile order

NUM_XCD = 8          # sfa_device.h: kNumXcd


def xcd_tile(ids, total):
    """sfa_device.h xcd_tile: dispatch id -> tile, XCD-contiguous ranges."""
    ids = np.asarray(ids)
    if total % NUM_XCD:
        return ids
    per = total // NUM_XCD
    return (ids % NUM_XCD) * per + ids // NUM_XCD


def lpt_seq_block(ids, total, nblk):
    """sfa_device.h lpt_seq_block: dispatch id -> (seq, blk, canon)."""
    tile = xcd_tile(ids, total)
    per = total // NUM_XCD
    if total % NUM_XCD == 0 and per % nblk == 0:
        k = per // nblk
        r = tile - (tile // per) * per
        seq = (tile // per) * k + r % k
        rank = r // k
    else:
        seq = tile // nblk
        rank = tile % nblk
    return seq, nblk - 1 - rank, seq * nblk + rank


def key_tile_order(ids, T, halves, nblk, nch):
    """sfa_bwd.hip key_tile_order: dispatch id -> (part, tile) of the key pass."""
    t = xcd_tile(ids, halves * T)
    if T % NUM_XCD:
        return (t >= T).astype(int), np.where(t >= T, t - T, t)
    h = T // NUM_XCD
    per = halves * h
    x, r = t // per, t % per
    part = (r >= h).astype(int)
    rr = r - part * h
    spx = h // (nblk * nch)
    tile = x * h + rr
    if spx * nblk * nch == h:
        rank, rem = rr // (spx * nch), rr % (spx * nch)
        tile = ((x * spx + rem // nch) * nblk + rank) * nch + rem % nch
    return part, tile


# ------------------------------------------------------------ slot table

def build_slots(window, lo, frac, merge=False):
    """sfa_api.hip build_slots: window distances then offsets, stable sort by
    lo; with merge, equal (lo, frac) neighbours become one slot.  Returns a
    list of (lo, frac, mult, rung)."""
    v = [(s, 0.0, -1) for s in range(window + 1)]
    v += [(int(l), float(np.float32(f)), k) for k, (l, f) in enumerate(zip(lo, frac))]
    v.sort(key=lambda x: x[0])  # Python's sort is stable
    out = []
    for l, f, r in v:
        if merge and out and out[-1][0] == l and out[-1][1] == f:
            out[-1] = (l, f, out[-1][2] + 1.0, -1)
            continue
        out.append((l, f, 1.0, r))
    check(len(out) <= MAX_SLOTS, "slot table over SFA_MAX_SLOTS")
    return out


# ------------------------------------------------------------ forward

def fwd_h16_shape(D, G):
    """sfa_fwd.hip fwd_h16_lpq / fwd_h16_bq: (lanes per query, queries per block)."""
    want = max(2 * G, D // 16)
    lpq = min(want, min(D // 2, 16))
    bq = 256 // lpq if lpq >= 8 else 64
    return lpq, bq


def forward(n, window, lo, frac, bq, interp=True):
    """Stages of fwd_offsets_kernel / fwd_offsets_h16_kernel for every query
    block: staged positions, the LDS rows each lane reads for each slot (row r
    and its interpolation partner r - 1) and the rotary rows.  Returns the
    number of (block, stage) pairs."""
    sl = build_slots(window, lo, frac, merge=True)
    S = len(sl)
    nblk = (n + bq - 1) // bq
    stages = 0
    for blk in range(nblk):
        i0 = blk * bq
        i_last = min(i0 + bq, n) - 1
        i = i0 + np.arange(bq)
        s = 0
        while s < S:
            lo0 = sl[s][0]
            if lo0 > i_last:
                break
            two = lambda t: 1 if (interp and sl[t][1] > 0.0) else 0
            lomax = lo0 + two(s)
            e = s + 1
            while e < S:
                le = sl[e][0]
                if le > i_last:
                    break
                need = max(lomax, le + two(e))
                if need - lo0 + bq > CAP:
                    break
                lomax = need
                e += 1
            r0 = i0 - lomax
            nrows = lomax - lo0 + bq
            check(0 < nrows <= CAP, "forward stage rows within the LDS capacity")
            pos = r0 + np.arange(nrows)
            loaded = (pos >= 0) & (pos < n)
            check(pos[loaded] < n, "staged rows (and their rotary rows) below n")
            for sj in range(s, e):
                l, f = sl[sj][0], sl[sj][1]
                r = i - l - r0
                check((r >= 0) & (r < nrows), "forward slot row inside the stage")
                if interp and f > 0.0:
                    check(r - 1 >= 0, "forward interpolation partner inside the stage")
                else:
                    check(r - 1 >= -1, "forward pad row")
            stages += 1
            s = e
    return stages


# ------------------------------------------------------------ query pass

def bwd_lpq(D, G):
    """sfa_bwd.hip bwd_lpq."""
    dims = 4 if G >= 4 else 8
    a = max(2 * G, D // dims)
    return min(min(a, D // 2), 16)


def bwd_bq(G):
    return 16 if G >= 4 else 64


def bwd_query_cap(G, esize=2, rpl=1):
    """sfa_bwd.hip bwd_query_cap: rows per query-pass stage."""
    if G >= 4:
        return 72
    if esize == 4:
        return CAP
    return 180 if rpl > 4 else 188


def bwd_query_lds(D, G, esize, rpl):
    """Bytes of LDS of a bwd_query workgroup: the K rows (fp32), the V rows
    (the input words), each array led by a pad row, the dd partials and the
    |dS| bound slots."""
    lpq, bq = bwd_lpq(D, G), bwd_bq(G)
    cap = bwd_query_cap(G, esize, rpl)
    ks = D + 4
    ksv = D // 2 + 4 if esize == 2 else ks
    nwv = bq * lpq // 64
    return (cap + 1) * (ks + ksv) * 4 + nwv * max(rpl * (lpq // G), 1) * 4 + nwv * 4


def query_pass(n, window, lo, frac, D, G, want_dd=True, batch_kv=1, esize=2):
    """bwd_query_kernel: stages (slots with a second row: interpolated or dd),
    the LDS rows each query reads, the p / dp workspace offsets of the writer
    lanes and the dd partial indices (one launch per rung window)."""
    sl = build_slots(window, lo, frac)
    S = len(sl)
    n_rungs = len(lo)
    lpq, bq = bwd_lpq(D, G), bwd_bq(G)
    nd = lpq // G
    rpl_small = 1 if nd >= 16 else 16 // nd
    # no offset gradient: the RPL = 0 instantiation
    dd_on = want_dd and n_rungs > 0
    rpl = 0 if not dd_on else (rpl_small if n_rungs <= rpl_small * nd else 16)
    qcap = bwd_query_cap(G, esize, rpl)
    # a CU holds two workgroups of 64 queries (fewer than 4 heads per KV
    # head) or four of 16 at head dims up to 64; at 128 (bf16) a workgroup
    # fits on its own
    per_cu = (2 if G < 4 else 4) if D <= 64 else 1
    check(bwd_query_lds(D, G, esize, rpl) * per_cu <= 163840, "query-pass LDS per CU")
    windows = [0] if (not want_dd or n_rungs <= rpl * nd) else list(range(0, n_rungs, rpl * nd))
    nblk = (n + bq - 1) // bq
    tiles = nblk * batch_kv
    p_size = batch_kv * S * n * G  # floats per p (or dp) array
    for r0w in windows:
        dd_of = lambda t: want_dd and n_rungs > 0 and 0 <= sl[t][3] - r0w < rpl * nd
        for blk in range(nblk):
            i0 = blk * bq
            i_last = min(i0 + bq, n) - 1
            i = i0 + np.arange(bq)
            active = i < n
            s = 0
            while s < S:
                lo0 = sl[s][0]
                if lo0 > i_last:
                    break
                two = lambda t: 1 if (sl[t][1] > 0.0 or dd_of(t)) else 0
                lomax = lo0 + two(s)
                e = s + 1
                while e < S:
                    le = sl[e][0]
                    if le > i_last:
                        break
                    need = max(lomax, le + two(e))
                    if need - lo0 + bq > qcap:
                        break
                    lomax = need
                    e += 1
                r0 = i0 - lomax
                nrows = lomax - lo0 + bq
                check(0 < nrows <= qcap, "query-pass stage within the LDS capacity")
                for sj in range(s, e):
                    l, f, _, rung = sl[sj]
                    r = i - l - r0
                    check((r >= 0) & (r < nrows), "query-pass slot row inside the stage")
                    if f > 0.0 or dd_of(sj):
                        check(r - 1 >= 0, "query-pass second row inside the stage")
                    # the extreme (sequence, head) pairs bound every other
                    lo_idx = (sj * n + i[active]) * G
                    hi_idx = (((batch_kv - 1) * S + sj) * n + i[active]) * G + G - 1
                    check((lo_idx >= 0) & (hi_idx < p_size), "p / dp workspace offset")
                s = e
            # the workgroup's bound on |dS| (bf16, G >= 2), one per tile
            check(0 <= (batch_kv - 1) * nblk + blk < tiles, "dS bound index")
            if want_dd and n_rungs:
                r_last = r0w + min(n_rungs - r0w, rpl * nd) - 1
                check(r_last * tiles + tiles - 1 < n_rungs * tiles, "dd partial index")
    return len(windows)


# ------------------------------------------------------------ key passes

def key_chunk_h16(D, G):
    """sfa_bwd.hip key_chunk_h16: dims per bf16 key-pass tile."""
    return 32 if G >= 4 and D >= 32 else min(16, D)


def key_half_row_words(G, D):
    """sfa_bwd.hip key_half_row_words."""
    kc = key_chunk_h16(D, G)
    return 2 * kc + 4 if G == 1 else kc * ((G + 1) // 2) + 4


def key_half_cap(G, D):
    """sfa_bwd.hip key_half_cap."""
    cap = (163840 * (KB_H16 // 64) // 16) // (4 * key_half_row_words(G, D))
    return min(max(cap, KB_H16 + 12), KB_H16 + 64)


def key_step_table(sl, n):
    """sfa_bwd.hip make_step_table: the (slot, tap) steps in order as (delta,
    tap weight, first step of a slot); at most twice the slot capacity."""
    table = []
    for x in sl:
        lo, fr = x[0], x[1]
        d0 = min(lo, n)
        if fr > 0.0:
            table.append((d0, np.float32(1.0) - np.float32(fr), True))
            table.append((d0 + 1, np.float32(fr), False))
        else:
            table.append((d0, np.float32(1.0), True))
    check(len(table) <= 2 * MAX_SLOTS, "step table capacity")
    return table


def key_pass_h16(n, window, lo, frac, G, D=64, batch_kv=1):
    """key_half_body (bf16): stage bounds, the ring of staged query rows (slot
    (q - q0) mod kcap of query j0 + q), the ring slot each lane reads at each
    (slot, tap) step and that it holds query j + delta, and the clamped rows
    and plane offsets of the weight loads.  Returns the number of steps."""
    sl = build_slots(window, lo, frac)
    S = len(sl)
    table = key_step_table(sl, n)
    nsteps = len(table)
    kcap = key_half_cap(G, D)
    check(kcap * key_half_row_words(G, D) * 4 <= 163840, "key-pass LDS of a workgroup")
    KB = KB_H16
    nblk = (n + KB - 1) // KB
    tid = np.arange(KB)
    lo_c = [min(x[0], n) for x in sl]              # 2 min(lo, n) + taps - 1, halved back
    taps = [2 if x[1] > 0.0 else 1 for x in sl]
    p_size = batch_kv * S * n * G
    bq = bwd_bq(G)
    nq = (n + bq - 1) // bq
    steps = 0
    for blk in range(nblk):
        j0 = blk * KB
        j = j0 + tid
        # dK (G >= 2): the query rows whose dS bounds scale the weights
        ilo = max(j0 + max(sl[0][0], -n), 0)
        ihi = min(j0 + KB + min(sl[-1][0], n), n - 1)
        if G >= 2 and ilo <= ihi:
            check(0 <= ilo // bq <= ihi // bq < nq, "dS bound tiles inside the sequence")
        ring = np.full(kcap, -(10 ** 9), dtype=np.int64)  # query held by each ring slot
        q0, have_hi, first = 0, 0, True
        # the loader's weight loads run over every step of the table and
        # once more past the end (rows clamped to [0, n); the plane advances
        # on a slot's first step and stays once past the end; the last
        # sequence bounds the others)
        slot_of = [sj for sj in range(S) for _ in range(taps[sj])]
        tap_of = [tp for sj in range(S) for tp in range(taps[sj])]
        plane = -1
        for fstep in range(nsteps + 2):
            d, w, first_of_slot = table[min(fstep, nsteps - 1)]
            live = fstep < nsteps
            if live and first_of_slot:
                plane += 1
            if live:
                sj = slot_of[fstep]
                wt = np.float32(sl[sj][1]) if tap_of[fstep] else np.float32(1.0) - np.float32(sl[sj][1])
                check(plane == sj and d == lo_c[sj] + tap_of[fstep] and w == wt, "step record of its slot and tap")
            i = np.clip(j + d, 0, n - 1)
            check((0 <= plane < S) & np.all(plane * n * G + i * G >= 0) &
                  np.all(((batch_kv - 1) * S + plane) * n * G + i * G + G <= p_size), "key-pass weight load offset")
        s = 0
        while s < S:
            lo0 = lo_c[s]
            if j0 + lo0 > n - 1:
                break
            lomax, e = lo0, s
            while e < S:
                le = lo_c[e]
                if j0 + le > n - 1 or le - lo0 + KB + 1 > kcap:
                    break
                lomax = le
                e += 1
            check(e > s, "a stage holds at least one slot")
            r0 = j0 + lo0
            nrows = min(lomax - lo0 + KB + 1, n - r0)
            hi = lo0 + nrows - 1
            if first:
                q0, have_hi, first = lo0, lo0 - 1, False
            check(lo0 >= q0, "stages in increasing offset order")
            base = (lo0 - q0) % kcap
            fnew = max(lo0, have_hi + 1)
            nnew = hi - fnew + 1
            rows = np.arange(max(nnew, 0))
            slot = fnew - lo0 + rows + base
            check(slot < 2 * kcap, "ring slot before the wrap")
            slot = np.where(slot >= kcap, slot - kcap, slot)
            check((slot >= 0) & (slot < kcap), "ring slot of a staged row")
            rn = j0 + fnew
            check(rn + rows < n, "staged query rows below n")
            ring[slot] = rn + rows  # rows before the sequence are staged as zeros
            have_hi = max(have_hi, hi)
            ts = sum(taps[:s])
            te = ts + sum(taps[s:e])
            check(te <= nsteps and table[ts][2] and (te == nsteps or table[te][2]), "stage step range")
            t = ts
            for sj in range(s, e):
                for tap in range(taps[sj]):
                    delta = lo_c[sj] + tap
                    check(table[t][0] == delta, "step record delta")
                    t += 1
                    valid = (j + delta >= 0) & (j + delta < n)
                    soff = delta - lo0 + base
                    wrap = tid >= kcap - soff
                    rs = tid + soff - np.where(wrap, kcap, 0)
                    check((rs[valid] >= 0) & (rs[valid] < kcap), "ring slot of a step")
                    check(ring[rs[valid]] == (j + delta)[valid], "ring slot holds the step's query row")
                    if G >= 2:
                        check(((j + delta)[valid] >= ilo) & ((j + delta)[valid] <= ihi),
                              "dS bound covers every weight's query row")
                    steps += 1
            s = e
        check(np.all(j[j < n] < n), "dK rotary row")
    return steps


def key_block_f32(G, D):
    """sfa_bwd.hip key_block for float tensors."""
    return 128 if 2 * G * 16 * 4 <= 256 else 64


def fp32_key_rope_row(delta):
    """bwd_key_kernel: rotary row of a step, R(delta) for a past offset and
    R(|delta|)^T for a future (negative) one."""
    return np.where(delta >= 0, delta, -delta)


def key_pass_f32(n, window, lo, frac, G, D=64, rope_row=fp32_key_rope_row):
    """bwd_key_kernel (float32): stage bounds, staged rows, the LDS row and
    the rotary row of each valid step, the workspace offset of its loads."""
    sl = build_slots(window, lo, frac)
    S = len(sl)
    KB = key_block_f32(G, D)
    KCAP = KB + 48
    nblk = (n + KB - 1) // KB
    tid = np.arange(KB)
    steps = 0
    for blk in range(nblk):
        j0 = blk * KB
        j = j0 + tid
        activej = j < n
        s = 0
        while s < S:
            lo0 = sl[s][0]
            if j0 + lo0 > n - 1:
                break
            lomax, e = lo0, s
            while e < S:
                le = sl[e][0]
                if j0 + le > n - 1 or le - lo0 + KB + 1 > KCAP:
                    break
                lomax = le
                e += 1
            r0 = j0 + lo0
            nrows = min(lomax - lo0 + KB + 1, n - r0)
            check(0 < nrows <= KCAP, "fp32 key-pass stage within the LDS capacity")
            for sj in range(s, e):
                l, f = sl[sj][0], sl[sj][1]
                for tap in range(2 if f > 0.0 else 1):
                    i = j + l + tap
                    valid = activej & (i >= 0) & (i < n) & ((tap == 1) | (j > 0) | (f == 0.0))
                    delta = l + tap
                    row = j + delta - r0
                    check((row[valid] >= 0) & (row[valid] < nrows), "fp32 key-pass LDS row")
                    rr = rope_row(np.full(KB, delta))
                    check((rr[valid] >= 0) & (rr[valid] < n), "fp32 key-pass rotary row")
                    steps += 1
            s = e
    return steps
