#!/usr/bin/env python3
"""Throughput of the sparse fixed-offset attention hot path on one MI355X.

One step = one training pass of a page-1 attention layer with a learned
alpha: the rung offsets for alpha (host producer), the forward over the
window plus the 15 interpolated Fibonacci rungs (with LSE), and the backward
(dQ, dK, dV, dd and dtheta).  Shape: 32 sequences x 1024 tokens (32,768
tokens per batch), 8 query heads over 2 key/value heads, head dim 64, window
10, RoPE 1e4, bf16 tensors; products on f16 operands in the forward and the
key pass, on fp32 in the query pass, every sum in fp32.  Inputs are seeded N(0,1)
and rotate over four resident sets (336 MB, more than the 256 MB Infinity
Cache) so HBM, not the cache, serves them.

Prints ONE JSON line: queries/s of the whole step (value), the step's
algorithmic HBM GB/s, a roofline object for the dominant kernel (timed with
HIP events on its launch stream over the timed region, taken by the
dispatch itself as its start and end timestamps; only that kernel's launches
are recorded there, since recording every launch lengthens the step; the
per-kernel breakdown comes from a second pass of the same steps with every
launch recorded), the forward alone on
the fixed-alpha page-1 layer (window 8, integer rungs), and the fp64 CPU
oracle timed on a bounded sample of the same step on one core, and on the
whole batch over all host cores (one worker process per core, at most 16).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("sparse-attn fwd(+bwd) queries/sec and achieved HBM GB/s (% of peak), "
          "1024-ctx GQA")
HBM_PEAK_GBS = 8000.0
NSETS = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector peak (packed FMA counted)


def algorithmic_flops(B, n, hq, hkv, D, S, n_interp, n_dd=0):
    """FLOPs each kernel must do by definition, per launch: 2 S D per
    query-head for every dot product or weighted sum over the S slots (forward:
    logits and the value sum; query pass: logits, dp and dq; each key-pass
    pass: dK and dV), plus 6 D per (KV head, query, interpolated rung) for the
    row interpolation (the key pass interpolates both its gathers), plus, for
    the offset gradient, 4 D per query-head and rung (q~ . dK and dO . dV)."""
    qh = B * n * hq
    lerp = 6 * D * n_interp * B * n * hkv
    return {
        "fwd_offsets": 4 * S * D * qh + lerp,
        "bwd_query": 6 * S * D * qh + lerp + 4 * D * n_dd * qh,
        "bwd_key": 4 * S * D * qh + 2 * lerp,
        "bwd_reduce": 0,
    }


def algorithmic_bytes(B, n, hq, hkv, D, esize):
    """Bytes each kernel must move by definition (every tensor once).

    "step" is the metric's count for a training step: the forward reads Q, K,
    V and writes O and LSE; the backward reads Q, K, V, O, dO and LSE and
    writes dQ, dK and dV.  "step_without_o" leaves out the backward's read of
    O, which this backward does not need (rowsum(dO * O) is recomputed)."""
    q = B * n * hq * D * esize
    kv = B * n * hkv * D * esize
    lse = B * n * hq * 4
    return {
        # read Q, K, V; write O and LSE
        "fwd_offsets": q + 2 * kv + q + lse,
        # read Q, K, V, dO, LSE; write dQ
        "bwd_query": q + 2 * kv + q + lse + q,
        # read Q, dO, K, V; write dK, dV
        "bwd_key": 2 * q + 2 * kv + 2 * kv,
        "bwd_reduce": 0,
        # the step: forward + backward, each tensor once per pass
        "step": (q + 2 * kv + q + lse) + (q + 2 * kv + q + q + lse + q + 2 * kv),
        "step_without_o": (q + 2 * kv + q + lse) + (q + 2 * kv + q + lse + q + 2 * kv),
        # forward without LSE
        "fwd_only": q + 2 * kv + q,
    }


KERNEL_SOURCES = ("fixed_offset_gather_amd/csrc/sfa_bwd.hip", "fixed_offset_gather_amd/csrc/sfa_fwd.hip",
                  "fixed_offset_gather_amd/csrc/sfa_device.h", "fixed_offset_gather_amd/csrc/sfa_internal.h")


def kernel_source_hash():
    """sha256 over the kernel sources, to tell whether counters still apply."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy of known size), or
    None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "%s__page1_learned_step__traffic.txt" % kernel)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return int(fields["hbm_bytes_per_launch"])


def measured_valu_busy(kernel):
    """VALU-busy percent of `kernel` from the committed counter summary
    (rocprofv3's derived VALUBusy counter), or None when there is none or the
    kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "%s__page1_learned_step__valu_busy.txt" % kernel)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash() or "valu_busy_pct" not in fields:
        return None
    return float(fields["valu_busy_pct"])


def calibration_copy():
    """One plain device copy of 256 MiB (outside any timed region), so a
    counter run sees a kernel of known traffic: it reads and writes 256 MiB."""
    import torch
    a = torch.empty(128 * 1024 * 1024, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def copy_bandwidth_gbs(reps=5):
    """The box's plain device-to-device copy rate (1 GiB read and 1 GiB
    written per copy, best of `reps`), outside any timed region: the HBM
    rate a streaming kernel can reach here, beside the 8 TB/s peak."""
    import torch
    a = torch.empty(512 * 1024 * 1024, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    nbytes = 2 * a.numel() * a.element_size()
    del a, b
    return round(nbytes / best / 1e9, 1)


def cpu_baseline(w, alpha, seqs, min_seconds=10.0, max_passes=3):
    """The fp64 oracle on `seqs` sequences of the same step, one thread,
    repeated until at least `min_seconds` of work (at most `max_passes`)."""
    from threadpoolctl import threadpool_limits

    import synth_inputs as si
    from oracle import attention as ref
    from oracle import offsets as ref_off

    q, k, v = si.qkv(seqs, w["seqlen"], w["hq"], w["hkv"], w["head_dim"], w["dtype"])
    do = si.upstream(seqs, w["seqlen"], w["hq"], w["head_dim"], w["dtype"])
    f = [si.to_f64(t) for t in (q, k, v, do)]
    dt, passes = 0.0, 0
    with threadpool_limits(limits=1):
        while passes < max_passes and (passes == 0 or dt < min_seconds):
            t0 = time.perf_counter()
            lo, frac = ref_off.rung_offsets(alpha)
            ref.forward(f[0], f[1], f[2], w["window"], lo, frac, w["rope_theta"])
            g = ref.backward(*f, w["window"], lo, frac, w["rope_theta"])
            ref.dtheta_from_dd(g["dd"], ref_off.FIB_BASE, alpha)
            dt += time.perf_counter() - t0
            passes += 1
    return {
        "value": passes * seqs * w["seqlen"] / dt,
        "unit": "queries/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "%d of %d sequences of the same step (forward + backward, fp64 numpy, one thread), "
                  "%d pass(es), %.1f s" % (seqs, w["batch"], passes, dt),
    }


def _oracle_worker(job):
    """One all-core baseline worker (a fresh process): the fp64 oracle step
    on sequences [a, b) of the seeded batch, one thread; returns seconds."""
    wname, alpha, a, b = job
    from threadpoolctl import threadpool_limits

    import synth_inputs as si
    from oracle import attention as ref
    from oracle import offsets as ref_off

    w = si.WORKLOADS[wname]
    q, k, v = si.qkv(w["batch"], w["seqlen"], w["hq"], w["hkv"], w["head_dim"], w["dtype"])
    do = si.upstream(w["batch"], w["seqlen"], w["hq"], w["head_dim"], w["dtype"])
    f = [si.to_f64(t[a:b]) for t in (q, k, v, do)]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        lo, frac = ref_off.rung_offsets(alpha)
        ref.forward(f[0], f[1], f[2], w["window"], lo, frac, w["rope_theta"])
        g = ref.backward(*f, w["window"], lo, frac, w["rope_theta"])
        ref.dtheta_from_dd(g["dd"], ref_off.FIB_BASE, alpha)
        return time.perf_counter() - t0


def cpu_baseline_all_cores(wname, alpha, batch, seqlen):
    """The same oracle step on every sequence of the batch, spread over the
    host's cores (at most 16 worker processes, started by spawn)."""
    import multiprocessing as mp
    cores = min(len(os.sched_getaffinity(0)), 16, batch)
    per = (batch + cores - 1) // cores
    jobs = [(wname, alpha, a, min(a + per, batch)) for a in range(0, batch, per)]
    with mp.get_context("spawn").Pool(len(jobs)) as pool:
        secs = pool.map(_oracle_worker, jobs)
    t = max(secs)
    return {
        "value": batch * seqlen / t,
        "unit": "queries/s",
        "cores": len(jobs),
        "kind": "oracle",
        "sample": "all %d sequences of the step, %d worker processes of one thread each (%d sequences each); "
                  "slowest worker %.1f s" % (batch, len(jobs), per, t),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=32)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (for counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    # The all-core oracle leg starts its worker processes here, before this
    # process touches the GPU, and ends them before the GPU work begins.
    if not args.no_cpu_baseline:
        import synth_inputs as si
        wl = si.WORKLOADS["page1_learned_step"]
        all_cores = cpu_baseline_all_cores("page1_learned_step", si.learned_alpha(), wl["batch"], wl["seqlen"])
        log("cpu baseline (all cores):", all_cores)

    import numpy as np
    import torch

    import fixed_offset_gather_amd as sfa
    import synth_inputs as si

    dev = torch.device("cuda:0")
    w = si.WORKLOADS["page1_learned_step"]
    B, n, hq, hkv, D = w["batch"], w["seqlen"], w["hq"], w["hkv"], w["head_dim"]
    W = w["window"]
    alpha = si.learned_alpha()
    base = sfa.base_fib()
    rope = sfa.rope_table_device(n, D, w["rope_theta"], dev)

    sets = []
    for s in range(NSETS):
        q, k, v = si.qkv(B, n, hq, hkv, D, w["dtype"], seed=si.SEED + 10 * s)
        do = si.upstream(B, n, hq, D, w["dtype"], seed=si.SEED + 10 * s)
        sets.append(tuple(t.to(dev) for t in (q, k, v, do)))
    lo, frac = sfa.offsets_fib(alpha)
    o_buf = torch.empty_like(sets[0][0])
    lse_buf = torch.empty((B, hq, n), dtype=torch.float32, device=dev)
    ws = torch.empty(sfa.bwd_workspace_bytes(sets[0][0], sets[0][1], W, lo, frac, rope),
                     dtype=torch.uint8, device=dev)

    def step(t):
        q, k, v, do = sets[t % NSETS]
        lo_, frac_ = sfa.offsets_fib(alpha)
        o, lse = sfa.fwd(q, k, v, W, lo_, frac_, rope, out=o_buf, lse=lse_buf)
        return sfa.bwd(q, k, v, lse, do, W, lo_, frac_, rope, base=base, alpha=alpha, workspace=ws)

    # Python's cyclic garbage collector stays off through the GPU sections:
    # a generation-2 collection (tens of ms once the process holds torch and
    # the oracle's objects) landing in a timed loop would be charged to the
    # kernels.  Reference counting still frees everything the loops drop.
    gc.collect()
    gc.disable()
    if args.calibrate_copy:
        calibration_copy()
    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    # Per-kernel breakdown: the same number of steps with every launch timed
    # by HIP events on its stream.  With every kernel recorded the step runs
    # longer and each kernel's average reads higher than with that kernel
    # alone selected (page-1 query pass 139 against 129 us), so this pass is
    # not the timed one.
    sfa.profile_reset()
    sfa.profile_enable(True)
    for t in range(args.steps):
        step(t)
    torch.cuda.synchronize()
    sfa.profile_enable(False)
    kern = {}
    for name in ("fwd_offsets", "bwd_query", "bwd_key", "bwd_reduce"):
        ms, cnt = sfa.profile_read(name)
        if cnt:
            kern[name] = {"avg_us": 1e3 * ms / cnt, "launches": cnt}
    dom = max(kern, key=lambda k_: kern[k_]["avg_us"] * kern[k_]["launches"])

    # The timed region: K steps, HIP events only around the dominant kernel
    # (its average launch time for the roofline, measured live here).
    sfa.profile_reset()
    sfa.profile_enable(True, only=dom)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.steps):
        step(t)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sfa.profile_enable(False, only=None)
    dms, dcnt = sfa.profile_read(dom)
    dom_us = 1e3 * dms / dcnt
    ms_per_step = 1e3 * wall / args.steps
    esize = 2
    ab = algorithmic_bytes(B, n, hq, hkv, D, esize)
    step_gbs = ab["step"] / (ms_per_step * 1e-3) / 1e9

    # Median of event-timed steps (torch's events on the stream the library
    # launches on), at least 100 of them, beside the wall-clock mean above.
    nev = max(100, args.steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nev)]
    torch.cuda.synchronize()
    for t in range(nev):
        evs[t][0].record()
        step(t)
        evs[t][1].record()
    torch.cuda.synchronize()
    step_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    step_events = {
        "iterations": nev,
        "median_ms": round(step_ms[nev // 2], 5),
        "p10_ms": round(step_ms[nev // 10], 5),
        "p90_ms": round(step_ms[(9 * nev) // 10], 5),
        "median_queries_per_s": round(B * n / (step_ms[nev // 2] * 1e-3), 1),
        "median_algorithmic_GBs": round(ab["step"] / (step_ms[nev // 2] * 1e-3) / 1e9, 1),
    }
    log("kernel avg us:", {k_: round(v_["avg_us"], 2) for k_, v_ in kern.items()},
        "step ms %.4f" % ms_per_step, "%s in the timed region %.2f us" % (dom, dom_us))

    dom_gbs = ab[dom] / (dom_us * 1e-6) / 1e9
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": round(dom_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(dom),
        "algorithmic_bytes_per_launch": ab[dom],
        "avg_launch_us": round(dom_us, 3),
    }
    # The same launch against the fp32 vector (VALU) peak: by arithmetic
    # intensity the backward kernels sit above the machine balance
    # (157.3 TFLOP/s / 8 TB/s), so this is the roofline that binds them.
    n_interp = sum(1 for f_ in frac if f_ > 0.0)
    af = algorithmic_flops(B, n, hq, hkv, D, W + 1 + len(lo), n_interp, n_dd=len(lo))
    dom_tf = af[dom] / (dom_us * 1e-6) / 1e12
    roofline["alu"] = {
        "achieved": round(dom_tf, 2),
        "peak": VALU_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(dom_tf / VALU_PEAK_TFLOPS, 4),
        "flops_per_launch": af[dom],
        "slots": W + 1 + len(lo),
        "interpolated_rungs": n_interp,
        "valu_busy_pct": measured_valu_busy(dom),
    }

    # Forward alone on the fixed-alpha page-1 layer (window 8, integer rungs).
    wf = si.WORKLOADS["page1_fixed"]
    lo1, frac1 = sfa.offsets_fib(wf["alpha"])
    for t in range(args.warmup):
        q, k, v, _ = sets[t % NSETS]
        sfa.fwd(q, k, v, wf["window"], lo1, frac1, rope, out=o_buf)
    torch.cuda.synchronize()
    sfa.profile_reset()
    sfa.profile_enable(True)
    t0 = time.perf_counter()
    for t in range(args.steps):
        q, k, v, _ = sets[t % NSETS]
        sfa.fwd(q, k, v, wf["window"], lo1, frac1, rope, out=o_buf)
    torch.cuda.synchronize()
    fwall = time.perf_counter() - t0
    sfa.profile_enable(False)
    fms, fcnt = sfa.profile_read("fwd_offsets")
    f_us = 1e3 * fms / max(fcnt, 1)
    fwd_only = {
        "workload": "page1_fixed",
        "queries_per_s": round(B * n / (f_us * 1e-6), 1),
        "avg_launch_us": round(f_us, 3),
        "wall_ms_per_call": round(1e3 * fwall / args.steps, 4),
        "algorithmic_GBs": round(ab["fwd_only"] / (f_us * 1e-6) / 1e9, 1),
        "frac_of_hbm_peak": round(ab["fwd_only"] / (f_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
    }

    # Learned interpolated gather against fused integer offsets (the pages'
    # one speed claim: learned about 5x slower at identical FLOPs), page-1
    # layer forward on the same inputs.  W = 0: self + 15 rungs on both
    # sides, no duplicate rows.  W = 8: the page's layer, where integer
    # rungs 1, 2, 3, 5, 8 coincide with window slots and are merged.
    def time_fwd(W_, lo_, fr_, interp=False, n_=n, rope_=None):
        # n_ != n: the same resident tokens as B * n / n_ sequences of n_
        rope_ = rope if rope_ is None else rope_
        B_ = B * n // n_
        shp_q, shp_kv = (B_, n_, hq, D), (B_, n_, hkv, D)
        ob = o_buf.view(shp_q)

        def call(t):
            q, k, v, _ = sets[t % NSETS]
            sfa.fwd(q.view(shp_q), k.view(shp_kv), v.view(shp_kv), W_, lo_, fr_, rope_, out=ob,
                    interp_kernel=interp)

        for t in range(args.warmup):
            call(t)
        torch.cuda.synchronize()
        sfa.profile_reset()
        sfa.profile_enable(True)
        for t in range(args.steps):
            call(t)
        torch.cuda.synchronize()
        sfa.profile_enable(False)
        ms_, c_ = sfa.profile_read("fwd_offsets")
        return round(1e3 * ms_ / max(c_, 1), 3)

    lo_l, fr_l = sfa.offsets_fib(alpha)
    rows = {
        "integer_w0": {"window": 0, "alpha": 1.0, "slots": 16, "avg_us": time_fwd(0, lo1, frac1)},
        "integer_w0_interp_kernel": {"window": 0, "alpha": 1.0, "slots": 16,
                                     "avg_us": time_fwd(0, lo1, frac1, interp=True)},
        "learned_w0": {"window": 0, "alpha": alpha, "slots": 16, "avg_us": time_fwd(0, lo_l, fr_l)},
        "integer_w8": {"window": 8, "alpha": 1.0, "slots": 24, "distinct_rows": 19,
                       "avg_us": time_fwd(8, lo1, frac1)},
        "learned_w8": {"window": 8, "alpha": alpha, "slots": 24, "avg_us": time_fwd(8, lo_l, fr_l)},
    }
    integer_vs_learned = {
        "workload": "page-1 layer forward (32 x 1024, 8/2 heads, D 64, bf16, RoPE 1e4)",
        "rows": rows,
        "learned_over_integer_w0": round(rows["learned_w0"]["avg_us"] / rows["integer_w0"]["avg_us"], 3),
        "learned_over_integer_w8": round(rows["learned_w8"]["avg_us"] / rows["integer_w8"]["avg_us"], 3),
        "pages_claim": "learned interpolated gather about 5x slower than fused integer offsets, no hardware stated",
    }
    log("integer vs learned:", {k_: v_["avg_us"] for k_, v_ in rows.items()})

    # Length extrapolation: the page-1 layer forward (W = 8) at longer
    # contexts with unchanged offsets, 32,768 tokens per batch throughout.
    lengths = {}
    for n_ in (1024, 2048, 4096, 8192):
        rope_ = sfa.rope_table_device(n_, D, w["rope_theta"], dev)
        row = {"batch": B * n // n_}
        for label, (lo_, fr_) in (("integer", (lo1, frac1)), ("learned", (lo_l, fr_l))):
            us = time_fwd(8, lo_, fr_, n_=n_, rope_=rope_)
            row[label] = {"avg_us": us, "queries_per_s": round(B * n / (us * 1e-6), 1),
                          "algorithmic_GBs": round(ab["fwd_only"] / (us * 1e-6) / 1e9, 1)}
        lengths[str(n_)] = row
        del rope_
    log("length extrapolation us:", {k_: (v_["integer"]["avg_us"], v_["learned"]["avg_us"])
                                     for k_, v_ in lengths.items()})

    # The staggered page-1 forward over 16 layers: W in {6, 8, 10, 12} with
    # the coprime schedule (16 alphas each), the power-of-2 base at W = 8
    # under the same schedule and the plain alpha = 1 control: 81 calls.
    ws_ = si.WORKLOADS["page1_staggered"]
    c2 = []
    for W_ in ws_["windows"]:
        for layer in range(ws_["layers"]):
            c2.append((W_, "fib", sfa.stagger_alpha("coprime", layer, ws_["layers"], ws_["stride"])))
    for layer in range(ws_["layers"]):
        c2.append((8, "pow2", sfa.stagger_alpha("coprime", layer, ws_["layers"], ws_["stride"])))
    c2.append((8, "pow2", 1.0))
    c2_us = []
    for W_, basis, a_ in c2:
        lo_c, fr_c = (sfa.offsets_fib if basis == "fib" else sfa.offsets_pow2)(a_)
        for t in range(2):
            q, k, v, _ = sets[t % NSETS]
            sfa.fwd(q, k, v, W_, lo_c, fr_c, rope, out=o_buf)
        torch.cuda.synchronize()
        sfa.profile_reset()
        sfa.profile_enable(True)
        for t in range(5):
            q, k, v, _ = sets[t % NSETS]
            sfa.fwd(q, k, v, W_, lo_c, fr_c, rope, out=o_buf)
        torch.cuda.synchronize()
        sfa.profile_enable(False)
        ms_, c_ = sfa.profile_read("fwd_offsets")
        c2_us.append(1e3 * ms_ / c_)
    c2_mean = sum(c2_us) / len(c2_us)
    staggered_forward = {
        "workload": "page1_staggered: 81 forward calls (16 coprime layers x W 6/8/10/12, power-of-2 base at W 8 "
                    "over the same 16 layers, alpha = 1 control), 32 x 1024, 8/2 heads, D 64, bf16, RoPE 1e4",
        "calls": len(c2_us),
        "mean_us_per_call": round(c2_mean, 3),
        "min_us": round(min(c2_us), 3),
        "max_us": round(max(c2_us), 3),
        "sum_us_all_calls": round(sum(c2_us), 1),
        "queries_per_s_per_call": round(B * n / (c2_mean * 1e-6), 1),
        "algorithmic_GBs": round(ab["fwd_only"] / (c2_mean * 1e-6) / 1e9, 1),
        "frac_of_hbm_peak": round(ab["fwd_only"] / (c2_mean * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "by_window_mean_us": {str(W_): round(sum(u for (w2, b2, _), u in zip(c2, c2_us) if w2 == W_ and b2 == "fib")
                                             / ws_["layers"], 3) for W_ in ws_["windows"]},
        "pow2_w8_mean_us": round(sum(u for (w2, b2, _), u in zip(c2, c2_us) if b2 == "pow2") / (ws_["layers"] + 1), 3),
    }
    log("staggered forward: mean %.2f us per call over %d calls" % (c2_mean, len(c2_us)))

    # Page 3's Christoffel layer trained: forward with LSE + backward (no
    # offset gradient) at context 2048, 8 x 2048 tokens, 4/4 heads, no
    # rotation; views of the resident tensors.  Causal: self + 128
    # carry-word offsets (m = 128, k = 1024).  Bidirectional by signed
    # offsets: self + -O and +O of the same m = 128, k = 1024 (257 slots).
    wc = si.WORKLOADS["ctx2048_christoffel"]
    Bc, nc, hc = wc["batch"], wc["seqlen"], wc["hq"]
    ne = Bc * nc * hc * D

    def cview(t):
        return t.view(-1)[:ne].view(Bc, nc, hc, D)

    lse_c = lse_buf.view(-1)[:Bc * hc * nc].view(Bc, hc, nc)

    def time_christoffel(offs, signed):
        fr0 = np.zeros(len(offs), dtype=np.float32)
        ws_c = torch.empty(sfa.bwd_workspace_bytes(cview(sets[0][0]), cview(sets[0][1]), 0, offs, fr0, None,
                                                   signed_offsets=signed), dtype=torch.uint8, device=dev)

        def cstep(t):
            q, k, v, do = (cview(x) for x in sets[t % NSETS])
            sfa.fwd(q, k, v, 0, offs, fr0, None, out=cview(o_buf), lse=lse_c, signed_offsets=signed)
            sfa.bwd(q, k, v, lse_c, do, 0, offs, fr0, None, workspace=ws_c, want_dd=False, signed_offsets=signed)

        for t in range(args.warmup):
            cstep(t)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(args.steps):
            cstep(t)
        torch.cuda.synchronize()
        cwall = time.perf_counter() - t0
        # per-kernel breakdown from a second pass with HIP events (not timed)
        sfa.profile_reset()
        sfa.profile_enable(True)
        for t in range(args.steps):
            cstep(t)
        torch.cuda.synchronize()
        sfa.profile_enable(False)
        ck = {}
        for name in ("fwd_offsets", "bwd_query", "bwd_key"):
            ms_, c_ = sfa.profile_read(name)
            if c_:
                ck[name] = round(1e3 * ms_ / c_, 3)
        S_ = 1 + len(offs)
        fwd_flops = 4 * S_ * D * Bc * nc * hc  # logits and value sum, 2 S D each per query-head
        fwd_bytes = 4 * ne * 2 + Bc * hc * nc * 4  # Q, K, V read, O written (bf16), LSE
        fu = ck.get("fwd_offsets", float("nan"))
        return {"slots": S_, "ms_per_step": round(1e3 * cwall / args.steps, 4),
                "queries_per_s": round(Bc * nc / (cwall / args.steps), 1), "kernels_avg_us": ck,
                "fwd_alu": {"flops_per_launch": fwd_flops, "achieved_TFLOPs": round(fwd_flops / (fu * 1e-6) / 1e12, 2),
                            "frac_of_valu_peak": round(fwd_flops / (fu * 1e-6) / 1e12 / VALU_PEAK_TFLOPS, 4)},
                "fwd_hbm": {"bytes_per_launch": fwd_bytes, "achieved_GBs": round(fwd_bytes / (fu * 1e-6) / 1e9, 1),
                            "frac_of_hbm_peak": round(fwd_bytes / (fu * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}

    christoffel_step = {
        "workload": "ctx2048_christoffel: 8 x 2048, 4/4 heads, D 64, bf16, no rotation, forward with LSE + "
                    "backward without dd",
        "causal_m128_k1024": time_christoffel(sfa.offsets_christoffel(wc["m"], wc["k"]), False),
        "bidirectional_signed_m128_k1024": time_christoffel(sfa.offsets_christoffel_signed(wc["m"], wc["k"]), True),
    }
    log("christoffel steps:", {k_: v_["ms_per_step"] for k_, v_ in christoffel_step.items() if k_ != "workload"})

    # Page 2's power-law layer trained: edge-list forward with LSE + its
    # backward (inverted table built once on the host), same shape.
    wp = si.WORKLOADS["ctx2048_powerlaw"]
    e_h, c_h = sfa.edges_powerlaw(wp["seqlen"], wp["radius"], wp["sigma"], wp["draws"], wp["width"], si.SEED)
    inv_h, ic_h = sfa.edges_transpose(e_h, c_h)
    ed, cd, invd, icd = (torch.from_numpy(x).to(dev) for x in (e_h, c_h, inv_h, ic_h))
    ws_p = torch.empty(sfa.bwd_edges_workspace_bytes(cview(sets[0][0]), cview(sets[0][1]), wp["width"]),
                       dtype=torch.uint8, device=dev)

    def pstep(t):
        q, k, v, do = (cview(x) for x in sets[t % NSETS])
        _, lse_ = sfa.fwd_edges(q, k, v, ed, cd, None, want_lse=True)
        sfa.bwd_edges(q, k, v, lse_, do, ed, cd, invd, icd, None, workspace=ws_p)

    for t in range(args.warmup):
        pstep(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.steps):
        pstep(t)
    torch.cuda.synchronize()
    pwall = time.perf_counter() - t0
    sfa.profile_reset()
    sfa.profile_enable(True)
    for t in range(args.steps):
        pstep(t)
    torch.cuda.synchronize()
    sfa.profile_enable(False)
    pk = {}
    for name in ("fwd_edges", "bwd_edges_query", "bwd_edges_key"):
        ms_, c_ = sfa.profile_read(name)
        if c_:
            pk[name] = round(1e3 * ms_ / c_, 3)
    fe_us = pk.get("fwd_edges", float("nan"))
    fe_bytes = 4 * ne * 2 + Bc * hc * nc * 4 + e_h.nbytes + c_h.nbytes  # Q, K, V, O, LSE and the lists
    powerlaw_step = {
        "workload": "ctx2048_powerlaw: 8 x 2048, 4/4 heads, D 64, bf16, 64-wide bidirectional edge lists "
                    "(mean %.1f keys), forward with LSE + backward" % float(c_h.mean()),
        "fwd_hbm": {"bytes_per_launch": int(fe_bytes), "achieved_GBs": round(fe_bytes / (fe_us * 1e-6) / 1e9, 1),
                    "frac_of_hbm_peak": round(fe_bytes / (fe_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "ms_per_step": round(1e3 * pwall / args.steps, 4),
        "queries_per_s": round(Bc * nc / (pwall / args.steps), 1),
        "kernels_avg_us": pk,
    }
    log("power-law step:", powerlaw_step["ms_per_step"], pk)
    del ws_p

    out = {
        "metric": METRIC,
        "value": round(B * n / (ms_per_step * 1e-3), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in/out; f16 and f32 operands; f32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": "page1_learned_step",
            "batch": B, "seqlen": n, "hq": hq, "hkv": hkv, "head_dim": D, "window": W,
            "rungs": "fibonacci x alpha (interpolated)", "alpha": alpha, "rope_theta": w["rope_theta"],
            "io_dtype": "bf16", "global_batch_tokens": B * n, "parallelism": "single-gpu",
        },
        "step_algorithmic_bytes": ab["step"],
        "step_algorithmic_GBs": round(step_gbs, 1),
        "step_frac_of_hbm_peak": round(step_gbs / HBM_PEAK_GBS, 4),
        "step_bytes_without_o_read": ab["step_without_o"],
        "step_events": step_events,
        # (not in counter runs: its copies would join the calibration copy's)
        "hbm_copy_GBs": None if args.calibrate_copy else copy_bandwidth_gbs(),
        "kernels_avg_us": {k_: round(v_["avg_us"], 3) for k_, v_ in kern.items()},
        "roofline": roofline,
        "fwd_only": fwd_only,
        "staggered_forward": staggered_forward,
        "integer_vs_learned": integer_vs_learned,
        "christoffel_step": christoffel_step,
        "powerlaw_step": powerlaw_step,
        "length_extrapolation": {"workload": "page-1 layer forward, W 8, 32,768 tokens per batch", "by_seqlen": lengths},
    }
    gc.enable()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, alpha, args.cpu_seqs)
        out["cpu_baseline_all_cores"] = all_cores
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
