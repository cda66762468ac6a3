#!/usr/bin/env python3
"""Decode-step benchmark of the indexer-selected sparse attention library.

One step = the whole hot path for one layer over the whole batch, i.e. one
sparse_attn_decode_step called as its launches as the library plans them
(sparse_attn_decode_step_stage): append the new token (K/V rows + FP8
projected key), the sampled selection bound, the scores of every position and
the kept candidates, the exact top-M per KV head, and gather-free sparse
attention over the selected rows.  At the 128K workload on a 256-CU MI355X
that is one launch (one workgroup per (batch row, KV head) unit).  Inputs are
synthetic (``workloads``) and resident in HBM before the timed region starts.

Prints ONE JSON line:
  value         decode steps/s (N=1 GPU; whole-job throughput)
  hbm_gbps      algorithmic bytes per step / step time
  roofline      the dominant kernel (the whole step at 128K) against 8 TB/s,
                and against this device's measured streaming-read rate
  cold_step_us  steps timed one at a time after a cache-evicting read
                (median, p10, p90, and per launch)
  cpu_baseline  the fp64 oracle on the host, on a bounded sample of units

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode steps/sec and achieved HBM GB/s at N=128K, M=2048, r=32"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
EVENT_EVERY = 4                       # timed steps between two bracketed dominant launches
RUN_LAUNCHES = 4                      # one-launch steps: back-to-back launches per event pair
DOMINANT_KERNEL = "unit_kernel"       # the dominant launch of the 128K step (one workgroup per unit)
KERNEL_SOURCES = ("indexer.hip", "device_common.hpp", "attend_common.hpp")
PLAN_NAMES = {0: "chunk_exact", 1: "filter", 2: "unit_workgroup", 3: "all_scores"}
STAGE_NAMES = {1: "SA_STEP_APPEND_BOUND", 2: "SA_STEP_CANDIDATES", 3: "SA_STEP_MERGE",
               4: "SA_STEP_ATTEND", 5: "SA_STEP_SELECT_ATTEND"}


def step_stages(sa, sh, wl):
    """The launches of one decode step as the library plans them for this
    shape on this device: (plan, [(name, stage, kernel)], algorithmic bytes
    per launch, name of the dominant launch).  With one workgroup per unit
    the whole step is one launch (append, bound, filter, merge, attention);
    with every position scored it is append + scores, then select + attend;
    otherwise it is append + bound, candidates, and select + attend."""
    plan = sa.sparse_attn_selection_plan(sh, wl.N, wl.M)
    ab = algorithmic_bytes(wl)
    if plan == sa.SA_PLAN_UNIT:
        stages = [("step", sa.SA_STEP_APPEND_BOUND, "unit_kernel")]
        return plan, stages, {"step": sum(ab.values())}, "step"
    if plan == sa.SA_PLAN_SCORES:
        # append + every position scored, then select + attend over the scores
        stages = [("append_score", sa.SA_STEP_APPEND_BOUND, "score_all_kernel"),
                  ("select_attend", sa.SA_STEP_SELECT_ATTEND, "scores_select_attend_kernel")]
        nbytes = {"append_score": ab["append_bound"] + ab["candidates"],
                  "select_attend": ab["select_attend"]}
        return plan, stages, nbytes, "select_attend"
    stages = [("append_bound", sa.SA_STEP_APPEND_BOUND, "append_bound_kernel"),
              ("candidates", sa.SA_STEP_CANDIDATES, "filter_kernel"),
              ("select_attend", sa.SA_STEP_SELECT_ATTEND, "select_attend_kernel")]
    return plan, stages, ab, "candidates"


def measure_baselines(sa, torch, inp, wl, sh, kp, idx, ws, timer, stream, reps, flush):
    """The JSSA article's two comparisons, on this GPU, outside the timed
    region: full attention over every cached row (its opening paragraph
    compares decoding throughput against it) and gather-then-attend ("Why
    token selection is not enough": the copy took more than half of the
    sparse-attention time at large batch) against the gather-free attention.
    Every timed call is preceded by an untimed 2 GiB read so that no call
    finds its rows left in the caches by the last."""
    from workloads import default_scale
    scale = default_scale(wl.d)
    dev = inp.q.device
    out = torch.empty(wl.B, wl.Hq, wl.d, dtype=torch.bfloat16, device=dev)
    dws = torch.empty(sa.sparse_attn_dense_workspace_size(sh, wl.N), dtype=torch.uint8,
                      device=dev)
    shg = sa.make_shape(wl.B, wl.Hq, wl.Hkv, wl.d, wl.r, wl.M)
    gws = torch.empty(sa.sparse_attn_dense_workspace_size(shg, wl.M), dtype=torch.uint8,
                      device=dev)
    Kg = torch.empty(wl.B, wl.Hkv, wl.M, wl.d, dtype=torch.bfloat16, device=dev)
    Vg = torch.empty_like(Kg)
    glens = inp.seq_lens.clamp(max=wl.M).to(torch.int32)
    calls = {
        "dense": lambda: sa.sparse_attn_dense_decode(sh, inp.q, inp.k_cache, inp.v_cache,
                                                     inp.seq_lens, wl.N, scale, out, None, dws),
        "gather_free": lambda: sa.sparse_attn_decode(sh, inp.q, inp.k_cache, inp.v_cache, idx,
                                                     wl.M, scale, out, None, ws),
        "gather": lambda: sa.sparse_attn_gather_kv(sh, idx, wl.M, inp.k_cache, inp.v_cache,
                                                   Kg, Vg),
        "contiguous": lambda: sa.sparse_attn_dense_decode(shg, inp.q, Kg, Vg, glens, wl.M,
                                                          scale, out, None, gws),
    }
    us = {}
    for name, call in calls.items():
        if name == "contiguous":                      # its input is the gathered copy
            calls["gather"]()
        call()
        pool = timer.create(2 * reps)
        for k in range(reps):
            flush()
            if name == "contiguous":
                calls["gather"]()
                flush()
            timer.record(pool[2 * k], stream)
            call()
            timer.record(pool[2 * k + 1], stream)
        torch.cuda.synchronize()
        us[name] = 1e3 * sum(timer.elapsed_ms(pool[2 * k], pool[2 * k + 1])
                             for k in range(reps)) / reps
        timer.destroy(pool)
    units = wl.B * wl.Hkv
    rows = units * wl.N * wl.d * 2 * 2
    sel = units * wl.M * wl.d * 2 * 2
    gather_then_attend = us["gather"] + us["contiguous"]
    return {
        "what": "full attention over all cached rows, and gather-then-attend, against this "
                "path (JSSA article: 6.43x over full attention at 128K / 2048 on B200; "
                "the copy took > 50% of the sparse-attention time)",
        "reps": reps,
        "dense_attention_us": round(us["dense"], 1),
        "dense_attention_gbps": round(rows / (us["dense"] * 1e-6) / 1e9, 1),
        "gather_free_attention_us": round(us["gather_free"], 2),
        "gather_us": round(us["gather"], 2),
        "contiguous_attention_us": round(us["contiguous"], 2),
        "gather_share_of_gather_then_attend": round(us["gather"] / gather_then_attend, 3),
        "gather_free_speedup_over_gather_then_attend":
            round(gather_then_attend / us["gather_free"], 2),
        "gather_gbps": round(2 * sel / (us["gather"] * 1e-6) / 1e9, 1),
    }


def _host_timed(torch, fn, reps):
    """Microseconds per call of fn on the host clock, synchronised on both
    sides of `reps` back-to-back calls (after two untimed ones)."""
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    return 1e6 * (time.perf_counter() - t0) / reps


def _step_calls(sa, sh, wl, x, kp, idx, out, ws, scale):
    """The decode step of inputs x as its launches (one call each)."""
    _, stages, _, _ = step_stages(sa, sh, wl)
    return [(lambda st=st: sa.sparse_attn_decode_step_stage(
        sh, st, x.pos, x.k_new, x.v_new, x.q, x.P, x.k_cache, x.v_cache, kp, x.seq_lens, wl.N,
        wl.M, scale, idx, out, None, ws)) for _, st, _ in stages]


def _cold_us(torch, timer, stream, fn, flusher, n):
    """Median, p10 and p90 microseconds of fn timed alone after a cache-evicting
    read each time (HIP events on the library's stream)."""
    import numpy as np
    fn()
    pool = timer.create(2 * n)
    for k in range(n):
        flusher()
        timer.record(pool[2 * k], stream)
        fn()
        timer.record(pool[2 * k + 1], stream)
    torch.cuda.synchronize()
    us = [1e3 * timer.elapsed_ms(pool[2 * k], pool[2 * k + 1]) for k in range(n)]
    timer.destroy(pool)
    return {"median_us": round(float(np.median(us)), 2),
            "p10_us": round(float(np.percentile(us, 10)), 2),
            "p90_us": round(float(np.percentile(us, 90)), 2), "steps": n}


def measure_small_workloads(sa, torch, dev, timer, stream, flusher, reps):
    """The decode step of the two single-layer workloads that fit in the 256 MB
    last-level cache -- gqa7_16k (B8 Hq28 Hkv4 N16384 M2048, 50.9 MB per step)
    and lisa_32k's sparse branch (B16 Hq32 Hkv8 N32768 M1024, 202.6 MB) --
    timed cold (each step after a 2 GiB read, so the bytes come from HBM)
    and back to back; GB/s of algorithmic bytes from the cold median."""
    from workloads import WORKLOADS, make_decode_inputs, default_scale
    res = {}
    for name in ("gqa7_16k", "lisa_32k"):
        wl = WORKLOADS[name]
        sh = sa.make_shape(wl.B, wl.Hq, wl.Hkv, wl.d, wl.r, wl.N)
        x = make_decode_inputs(wl, seed=0, device=dev)
        kp = torch.empty(wl.B, wl.Hkv, wl.N, wl.r, dtype=torch.uint8, device=dev)
        sa.sparse_attn_project_keys(sh, x.k_cache, x.P, 0, wl.N, kp)
        ws = sa.alloc_workspace(sh, wl.N, wl.M, device=dev)
        idx = torch.empty(wl.B, wl.Hkv, wl.M, dtype=torch.int32, device=dev)
        out = torch.empty(wl.B, wl.Hq, wl.d, dtype=torch.bfloat16, device=dev)
        calls = _step_calls(sa, sh, wl, x, kp, idx, out, ws, default_scale(wl.d))
        plan, stages, nbytes, _ = step_stages(sa, sh, wl)

        def step():
            for c in calls:
                c()
        cold = _cold_us(torch, timer, stream, step, flusher, reps)
        step_bytes = sum(nbytes.values())
        res[name] = {"plan": PLAN_NAMES.get(plan, str(plan)),
                     "launches": [k for _, _, k in stages],
                     "cold": cold, "back_to_back_us": round(_host_timed(torch, step, 3 * reps), 2),
                     "step_bytes": step_bytes,
                     "cold_hbm_gbps": round(step_bytes / (cold["median_us"] * 1e-6) / 1e9, 1)}
        del x, kp, ws
        torch.cuda.empty_cache()
    return res


def measure_extensions(sa, torch, dev, reps, timer=None, stream=None, flusher=None):
    """The two extensions at their own workloads, outside the timed region.

    Cross-layer index reuse (IndexCache pages: layers that reuse the indices
    of an earlier layer skip its indexer): eight layers of reuse8_64k with
    the indexer and top-M on layers 0 and 4 only, the other layers appending
    their token and attending over their source layer's indices, against the
    same eight layers each running the whole decode step.

    Gated hybrid (LISA items: a linear-attention branch merged with the
    sparse one through a gate): the decode step of lisa_32k followed by
    sparse_attn_linear_gate (state update and mix), against the decode step
    alone and against full attention over every cached row.  The linear state
    holds arbitrary values here (its cost does not depend on them).

    Both are timed back to back (host clock) and, with a flusher, cold (each
    eight-layer or hybrid step after a 2 GiB read)."""
    from workloads import WORKLOADS, make_decode_inputs, default_scale
    res = {}

    wl = WORKLOADS["reuse8_64k"]
    B, Hq, Hkv, d, N, r, M = wl.B, wl.Hq, wl.Hkv, wl.d, wl.N, wl.r, wl.M
    sh = sa.make_shape(B, Hq, Hkv, d, r, N)
    layers = [make_decode_inputs(wl, seed=0, layer=l, device=dev) for l in range(wl.layers)]
    kps = []
    for inp in layers:
        kp = torch.empty(B, Hkv, N, r, dtype=torch.uint8, device=dev)
        sa.sparse_attn_project_keys(sh, inp.k_cache, inp.P, 0, N, kp)       # prefill
        kps.append(kp)
    ws = sa.alloc_workspace(sh, N, M, device=dev)
    idx = [torch.empty(B, Hkv, M, dtype=torch.int32, device=dev) for _ in range(wl.layers)]
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    scale = default_scale(d)
    full_calls = [_step_calls(sa, sh, wl, layers[l], kps[l], idx[l], out, ws, scale)
                  for l in range(wl.layers)]

    def full(l):
        for c in full_calls[l]:
            c()

    def reused(l, src):
        x = layers[l]
        sa.sparse_attn_append_kv(sh, x.pos, x.k_new, x.v_new, x.P, x.k_cache, x.v_cache, kps[l])
        sa.sparse_attn_decode(sh, x.q, x.k_cache, x.v_cache, idx[src], M, scale, out, None, ws)

    def step_reuse():
        for l in range(wl.layers):
            src = max(f for f in wl.full_layers if f <= l)
            if l == src:
                full(l)
            else:
                reused(l, src)

    def step_every_layer():
        for l in range(wl.layers):
            full(l)

    t_reuse = _host_timed(torch, step_reuse, reps)
    t_all = _host_timed(torch, step_every_layer, reps)
    bk = algorithmic_bytes(wl)
    units = B * Hkv
    layer_full = sum(bk.values())
    layer_reused = (bk["append_bound"] + units * M * 4 + units * M * d * 2 * 2
                    + 2 * B * Hq * d * 2)                 # idx read, rows, q, out
    n_full = len(wl.full_layers)
    bytes_reuse = n_full * layer_full + (wl.layers - n_full) * layer_reused
    bytes_all = wl.layers * layer_full
    res["index_reuse"] = {
        "workload": "reuse8_64k: 8 layers of B%d Hq%d Hkv%d d%d N%d r%d M%d, indexer on layers %s"
                    % (B, Hq, Hkv, d, N, r, M, ",".join(map(str, wl.full_layers))),
        "reps": reps,
        "us_per_8_layer_step": round(t_reuse, 1),
        "us_per_8_layer_step_every_layer_indexed": round(t_all, 1),
        "speedup": round(t_all / t_reuse, 3),
        "bytes_per_8_layer_step": bytes_reuse,
        "bytes_per_8_layer_step_every_layer_indexed": bytes_all,
        "hbm_gbps": round(bytes_reuse / (t_reuse * 1e-6) / 1e9, 1),
    }
    if flusher is not None:
        cold = _cold_us(torch, timer, stream, step_reuse, flusher, reps)
        res["index_reuse"]["cold"] = cold
        res["index_reuse"]["cold_hbm_gbps"] = round(
            bytes_reuse / (cold["median_us"] * 1e-6) / 1e9, 1)
    del layers, kps, ws, idx, full_calls
    torch.cuda.empty_cache()

    wl = WORKLOADS["lisa_32k"]
    B, Hq, Hkv, d, N, r, M = wl.B, wl.Hq, wl.Hkv, wl.d, wl.N, wl.r, wl.M
    sh = sa.make_shape(B, Hq, Hkv, d, r, N)
    x = make_decode_inputs(wl, seed=0, device=dev)
    kp = torch.empty(B, Hkv, N, r, dtype=torch.uint8, device=dev)
    sa.sparse_attn_project_keys(sh, x.k_cache, x.P, 0, N, kp)
    ws = sa.alloc_workspace(sh, N, M, device=dev)
    dws = torch.empty(sa.sparse_attn_dense_workspace_size(sh, N), dtype=torch.uint8, device=dev)
    idx1 = torch.empty(B, Hkv, M, dtype=torch.int32, device=dev)
    o_sp = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(o_sp)
    S = torch.zeros(B, Hkv, d, d, dtype=torch.float32, device=dev)
    z = torch.ones(B, Hkv, d, dtype=torch.float32, device=dev)
    scale = default_scale(d)
    sparse_calls = _step_calls(sa, sh, wl, x, kp, idx1, o_sp, ws, scale)

    def sparse_step():
        for c in sparse_calls:
            c()

    def gate():
        sa.sparse_attn_linear_gate(sh, x.q, x.k_new.view(B, Hkv, d), x.v_new.view(B, Hkv, d),
                                   S, z, x.w_gate, o_sp, out, True)

    def hybrid_step():
        sparse_step()
        gate()

    t_sparse = _host_timed(torch, sparse_step, reps)
    t_hybrid = _host_timed(torch, hybrid_step, reps)
    t_dense = _host_timed(torch, lambda: sa.sparse_attn_dense_decode(
        sh, x.q, x.k_cache, x.v_cache, x.seq_lens, N, scale, o_sp, None, dws), reps)
    units = B * Hkv
    gate_bytes = (units * d * d * 4 * 2 + units * d * 4 * 2 + 2 * B * Hq * d * 2
                  + units * 2 * d * 2 + Hq * d * 4 + B * Hq * d * 2)
    hybrid_bytes = sum(algorithmic_bytes(wl).values()) + gate_bytes
    res["gated_hybrid"] = {
        "workload": "lisa_32k: B%d Hq%d Hkv%d d%d N%d r%d M%d, fp32 linear state %dx%d per KV "
                    "head" % (B, Hq, Hkv, d, N, r, M, d, d),
        "reps": reps,
        "us_per_hybrid_step": round(t_hybrid, 1),
        "us_per_sparse_step": round(t_sparse, 1),
        "us_full_attention": round(t_dense, 1),
        "hybrid_speedup_over_full_attention": round(t_dense / t_hybrid, 2),
        "bytes_per_hybrid_step": hybrid_bytes,
        "hbm_gbps": round(hybrid_bytes / (t_hybrid * 1e-6) / 1e9, 1),
    }
    if flusher is not None:
        cold = _cold_us(torch, timer, stream, hybrid_step, flusher, reps)
        res["gated_hybrid"]["cold"] = cold
        res["gated_hybrid"]["cold_hbm_gbps"] = round(
            hybrid_bytes / (cold["median_us"] * 1e-6) / 1e9, 1)
    return res


def algorithmic_bytes(wl):
    """Bytes the method itself must move per step, by call: every input read
    once and every output written once (workspace traffic is not counted)."""
    units = wl.B * wl.Hkv
    q = wl.B * wl.Hq * wl.d * 2
    idx = units * wl.M * 4
    P = wl.Hkv * wl.d * wl.r * 4
    # read the new K/V rows, write K/V rows + the FP8 projected key
    append = units * (2 * wl.d * 2) + units * (2 * wl.d * 2 + wl.r) + wl.B * 4 + P
    candidates = units * wl.N * wl.r + q + P       # the FP8 key stream, the queries, P
    # write the selected positions; read the selected K/V rows and the
    # queries, write the outputs
    select_attend = idx + units * wl.M * wl.d * 2 * 2 + q + wl.B * wl.Hq * wl.d * 2
    # the sampled bound reads a few rows again: no bytes of its own are required
    return {"append_bound": append, "candidates": candidates, "select_attend": select_attend}


def _source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_attention_long_kv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, src_hash):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel_key)
    if not e or e.get("source_hash") != src_hash:
        return None
    return e.get("bytes_per_launch")


CALIB_KERNEL_TAG = "neg"      # torch.neg on fp32: reads and writes exactly n*4 bytes


class HipTimer:
    """HIP timing events recorded on a raw stream.  They are created with
    hipEventDisableSystemFence: recording one then costs no cache write-back,
    so timing every call of a step does not slow the step down (the default
    events of torch.cuda.Event flush caches at each record)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        lib = None
        for name in ("libamdhip64.so.7", "libamdhip64.so"):
            try:
                lib = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if lib is None:
            raise RuntimeError("HIP runtime library not found")
        vp = ctypes.c_void_p
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [vp, vp]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        lib.hipEventDestroy.argtypes = [vp]
        self.lib = lib

    def create(self, n):
        evs = []
        for _ in range(n):
            e = self.ct.c_void_p()
            if self.lib.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            evs.append(e)
        return evs

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ev, self.ct.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.lib.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


def ingest_counters(fetch_csv, write_csv, calib_mib, kernel=DOMINANT_KERNEL):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE; both with --calibration-mib) into profiles/traffic.json: each
    counter's per-dispatch mean for `kernel`, scaled by what the same counter
    reads for the calibration kernel, whose true traffic is known."""
    import csv

    def per_dispatch(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        return vals

    def mean_for(vals, pred):
        xs = [v for (name, _), v in vals.items() if pred(name)]
        if not xs:
            raise SystemExit("no dispatch matched in the counter file")
        return sum(xs) / len(xs), len(xs)

    true_bytes = calib_mib * 2.0 ** 20
    out = {}
    for label, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"),
                                 ("write", write_csv, "WRITE_SIZE")):
        vals = per_dispatch(path, counter)
        calib, _ = mean_for(vals, lambda n: CALIB_KERNEL_TAG in n and "elementwise" in n)
        kern, n = mean_for(vals, lambda n: kernel in n)
        scale = true_bytes / (calib * 1024.0)
        out[label] = {"counter_kib_per_dispatch": kern, "dispatches": n,
                      "calibration_kib": calib, "scale": scale,
                      "bytes_per_launch": kern * 1024.0 * scale}
    src_hash = _source_hash(KERNEL_SOURCES)
    entry = {"source_hash": src_hash,
             "bytes_per_launch": round(out["fetch"]["bytes_per_launch"]
                                       + out["write"]["bytes_per_launch"]),
             "fetch": out["fetch"], "write": out["write"],
             "calibration": "torch.neg over %d MiB of fp32 (reads and writes %d MiB)"
                            % (calib_mib, calib_mib)}
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table[kernel] = entry
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1)
    print(json.dumps({kernel: entry}))


def cpu_baseline(inp, wl, n_units, min_seconds=10.0, seed=0):
    """Time the oracle on a bounded sample of (batch row, KV head) units.

    The sampled units' decode steps are repeated until enough oracle time has
    been measured, first one unit at a time on one thread (numpy/BLAS pinned
    to one thread), then with the units running concurrently on every host
    thread this process may use (at most 16: the host's share of one GPU),
    each call's BLAS still on one thread.  At least that many units are
    sampled, so every thread has its own.  Each unit's FP8 cache is prepared
    by the oracle beforehand, untimed: it is cache state, not part of the
    step.  The headline value is the all-threads rate; `cores` is the number
    of threads it used."""
    import concurrent.futures as cf
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from workloads import default_scale

    available = len(os.sched_getaffinity(0))
    threads = max(1, min(16, available))
    rng = np.random.default_rng(seed)
    units = rng.choice(wl.B * wl.Hkv, size=min(max(n_units, threads), wl.B * wl.Hkv),
                       replace=False)
    G = wl.G
    P64 = inp.P.double().cpu().numpy()
    q64 = inp.q.double().cpu().numpy()
    with threadpool_limits(limits=1):
        prepared = []
        for u in units:
            b, h = divmod(int(u), wl.Hkv)
            K = inp.k_cache[b, h].double().cpu().numpy()
            V = inp.v_cache[b, h].double().cpu().numpy()
            kp = oracle.project_keys(K, P64[h])            # cache state: not timed
            kn = inp.k_new[b, h].double().cpu().numpy()
            prepared.append((b, h, K, V, kp, kn))

        def one(item):
            b, h, K, V, kp, kn = item
            kp[wl.N - 1] = oracle.project_keys(kn, P64[h])[0]
            K[wl.N - 1] = kn[0]
            oracle.decode_step_unit(q64[b, h * G:(h + 1) * G], K, V, kp, P64[h], wl.N, wl.M,
                                    default_scale(wl.d))

        total, count = 0.0, 0
        while total < min_seconds or count < len(prepared):
            for item in prepared:
                t0 = time.perf_counter()
                one(item)
                total += time.perf_counter() - t0
                count += 1
        per_unit = total / count
        single = {"value": round(1.0 / (per_unit * wl.B * wl.Hkv), 4), "threads": 1,
                  "unit_steps": count, "seconds_measured": round(total, 2)}

        done, wall = 0, 0.0
        with cf.ThreadPoolExecutor(threads) as ex:
            while wall < min_seconds / 2 or done < len(prepared):
                t0 = time.perf_counter()
                list(ex.map(one, prepared))
                wall += time.perf_counter() - t0
                done += len(prepared)
        step_all = wall / done * wl.B * wl.Hkv
    return {"value": round(1.0 / step_all, 4), "unit": "steps/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of the %d (batch row, KV head) units of one step, run "
                      "concurrently on %d host threads (%d unit-steps in %.1f s of wall "
                      "clock), scaled to the whole step; numpy fp64, BLAS one thread per "
                      "call" % (len(prepared), wl.B * wl.Hkv, threads, done, wall),
            "seconds_measured": round(wall, 2),
            "cores_available": available,
            "single_thread": single,
            "cpu_model": _cpu_model()}


def _cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family/model/stepping
    numbers (some hosts report only a short model name) and the count of
    logical CPUs the machine has."""
    info, n = {}, 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    continue
                k, v = (x.strip() for x in line.split(":", 1))
                if k == "processor":
                    n += 1
                elif k not in info:
                    info[k] = v
    except OSError:
        return None
    name = info.get("model name", "unknown")
    return "%s (%s, family %s model %s stepping %s; %d logical CPUs on the host)" % (
        name, info.get("vendor_id", "?"), info.get("cpu family", "?"), info.get("model", "?"),
        info.get("stepping", "?"), n)


class ReadFlush:
    """A 2 GiB streaming read (sparse_attn_stream_read) that evicts the 256 MB
    last-level cache before a cold measurement (a read, not a write: a write
    flush leaves dirty lines whose write-back lands in the next launch)."""

    def __init__(self, sa, torch, dev):
        self.sa = sa
        self.buf = torch.empty(2 ** 31, dtype=torch.uint8, device=dev)
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def __call__(self):
        self.sa.sparse_attn_stream_read(self.buf, self.sink)


def cold_steps(timer, stream, calls, names, flusher, n):
    """Steps timed one at a time, each after a cache-evicting read: median,
    p10, p90 of the step and the median of each launch (microseconds)."""
    import numpy as np
    n_ev = len(calls) + 1
    pool = timer.create(n_ev * n)
    for k in range(n):
        flusher()
        rec = pool[k * n_ev:(k + 1) * n_ev]
        for i, call in enumerate(calls):
            timer.record(rec[i], stream)
            call()
        timer.record(rec[-1], stream)
    import torch
    torch.cuda.synchronize()
    per = [[1e3 * timer.elapsed_ms(pool[k * n_ev + i], pool[k * n_ev + i + 1])
            for i in range(len(calls))] for k in range(n)]
    us = [1e3 * timer.elapsed_ms(pool[k * n_ev], pool[k * n_ev + n_ev - 1]) for k in range(n)]
    timer.destroy(pool)
    q10, q50, q90 = (float(np.percentile(us, p)) for p in (10, 50, 90))
    return {"steps": n, "read_flush_mib": 2048, "median_us": round(q50, 2),
            "p10_us": round(q10, 2), "p90_us": round(q90, 2),
            "median_us_per_call": {k: round(float(np.median([r[i] for r in per])), 2)
                                   for i, k in enumerate(names)}}


def stream_read_gbps(sa, torch, dev, timer, stream, reps=10):
    """This device's streaming-read rate: one read of 1 GiB with the fastest
    pattern measured here (sparse_attn_stream_read), GB/s averaged over reps."""
    rbuf = torch.empty(2 ** 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        sa.sparse_attn_stream_read(rbuf, sink)
    pool = timer.create(2 * reps)
    for k in range(reps):
        timer.record(pool[2 * k], stream)
        sa.sparse_attn_stream_read(rbuf, sink)
        timer.record(pool[2 * k + 1], stream)
    torch.cuda.synchronize()
    us = 1e3 * sum(timer.elapsed_ms(pool[2 * k], pool[2 * k + 1]) for k in range(reps)) / reps
    timer.destroy(pool)
    return 2 ** 30 / (us * 1e-6) / 1e9


def row_read_gbps(sa, torch, sh, idx, wl, inp, timer, stream, flusher, reps=5):
    """The selected K and V rows (the step's idx) read alone, after a
    cache-evicting read each time: into registers with the attention's lane
    layout, and straight into LDS.  GB/s of the rows' bytes."""
    sink = torch.zeros(1, dtype=torch.int32, device=inp.q.device)
    valid = int((idx >= 0).sum().item())
    nbytes = valid * wl.d * 2 * 2
    res = {}
    for mode, name in ((0, "registers"), (1, "lds")):
        sa.sparse_attn_row_read(sh, idx, wl.M, inp.k_cache, inp.v_cache, mode, sink)
        pool = timer.create(2 * reps)
        for k in range(reps):
            flusher()
            timer.record(pool[2 * k], stream)
            sa.sparse_attn_row_read(sh, idx, wl.M, inp.k_cache, inp.v_cache, mode, sink)
            timer.record(pool[2 * k + 1], stream)
        torch.cuda.synchronize()
        us = 1e3 * sum(timer.elapsed_ms(pool[2 * k], pool[2 * k + 1])
                       for k in range(reps)) / reps
        timer.destroy(pool)
        res[name] = {"us": round(us, 2), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)}
    res["bytes"] = nbytes
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="longctx_128k")
    ap.add_argument("--cpu-units", type=int, default=16,
                    help="units of the step timed for the oracle baseline (0 = skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="steps timed one by one after a 2 GiB read flush, after the "
                         "timed region (0: skip)")
    ap.add_argument("--ext-reps", type=int, default=10,
                    help="steps timed per extension workload (index reuse over eight "
                         "layers, gated hybrid); 0: skip them")
    ap.add_argument("--baseline-reps", type=int, default=5,
                    help="calls timed per comparison baseline (0: skip them)")
    ap.add_argument("--calibration-mib", type=int, default=0,
                    help="before the timed region, run one torch.neg over this many MiB "
                         "(a kernel of known traffic for scaling rocprofv3 byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: write profiles/traffic.json from two rocprofv3 "
                         "--pmc counter files of a --calibration-mib run")
    a = ap.parse_args(argv)

    if a.traffic_from:
        ingest_counters(a.traffic_from[0], a.traffic_from[1], a.calibration_mib or 1024)
        return

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every step of this path is independent per "
              "(batch row, KV head) unit and this benchmark measures a single MI355X; "
              "--gpus %d is not supported." % a.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_long_kv_amd as sa
    from workloads import WORKLOADS, make_decode_inputs, default_scale

    wl = WORKLOADS[a.workload]
    if wl.layers != 1:
        raise SystemExit("bench.py times single-layer workloads")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sa.load()
    print("bench: generating %s inputs" % wl.name, file=sys.stderr, flush=True)
    inp = make_decode_inputs(wl, seed=a.seed, device="cuda")
    sh = sa.make_shape(wl.B, wl.Hq, wl.Hkv, wl.d, wl.r, wl.N)
    kp = torch.empty(wl.B, wl.Hkv, wl.N, wl.r, dtype=torch.uint8, device=dev)
    sa.sparse_attn_project_keys(sh, inp.k_cache, inp.P, 0, wl.N, kp)     # prefill (untimed)
    ws = sa.alloc_workspace(sh, wl.N, wl.M, device=dev)
    idx = torch.empty(wl.B, wl.Hkv, wl.M, dtype=torch.int32, device=dev)
    out = torch.empty(wl.B, wl.Hq, wl.d, dtype=torch.bfloat16, device=dev)
    scale = default_scale(wl.d)
    torch.cuda.synchronize()

    # the launches of sparse_attn_decode_step, one call each, as the library
    # plans them for this shape and device
    plan, stages, bytes_k, dom = step_stages(sa, sh, wl)
    names = tuple(n for n, _, _ in stages)
    ev = {k: [] for k in names}
    lse = None

    def stage(st):
        return lambda: sa.sparse_attn_decode_step_stage(
            sh, st, inp.pos, inp.k_new, inp.v_new, inp.q, inp.P, inp.k_cache, inp.v_cache, kp,
            inp.seq_lens, wl.N, wl.M, scale, idx, out, lse, ws)
    calls = tuple(stage(st) for _, st, _ in stages)

    timer = HipTimer()
    stream = torch.cuda.current_stream(dev).cuda_stream    # the stream every call launches on
    dom_i = names.index(dom)

    def step(rec, every_call=False):
        # rec: this step's events.  In the timed region only the dominant call
        # is bracketed (two events), in every EVENT_EVERY-th step; the
        # breakdown pass brackets every call.
        for i, call in enumerate(calls):
            if rec is not None and (every_call or i == dom_i):
                timer.record(rec[i if every_call else 0], stream)
            call()
            if rec is not None and not every_call and i == dom_i:
                timer.record(rec[1], stream)
        if rec is not None and every_call:
            timer.record(rec[-1], stream)
            for i, k in enumerate(names):
                ev[k].append((rec[i], rec[i + 1]))
        elif rec is not None:
            dom_ev.append((rec[0], rec[1], 1))

    print("bench: warmup %d" % a.warmup, file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        step(None)
    if a.calibration_mib > 0:
        x = torch.ones(a.calibration_mib * 2 ** 18, dtype=torch.float32, device=dev)
        torch.neg(x, out=torch.empty_like(x))
        del x
    torch.cuda.synchronize()

    # timed region: exactly K steps, back to back, synchronised on both sides.
    # The events for it are created beforehand (creating them is host work
    # that would otherwise sit in the timed region while the GPU waits).
    # HIP events time the dominant launch.  An event pair costs the GPU time
    # of its own (~1.5-2 us per bracketed launch here, against rocprofv3's
    # durations), so pairs are sparse: when the step is that one launch, a
    # pair brackets a run of RUN_LAUNCHES back-to-back launches in every
    # 2 RUN_LAUNCHES steps; otherwise it brackets the dominant call of every
    # EVENT_EVERY-th step.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    one_launch = len(calls) == 1
    run = RUN_LAUNCHES if one_launch else 1
    period = 2 * RUN_LAUNCHES if one_launch else EVENT_EVERY
    dom_ev = []                                 # (start event, end event, launches)
    pool = timer.create(2 * ((a.steps + period - 1) // period))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(a.steps):
        j, r = divmod(k, period)
        if not one_launch:
            step(pool[2 * j:2 * j + 2] if r == 0 else None)
            continue
        if r == 0:
            timer.record(pool[2 * j], stream)
        calls[0]()
        if r == run - 1 or (r < run and k == a.steps - 1):
            timer.record(pool[2 * j + 1], stream)
            dom_ev.append((pool[2 * j], pool[2 * j + 1], r + 1))
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(end)
    ms_per_step = 1e3 * wall / a.steps          # host clock around the K steps
    dom_launches = sum(n for _, _, n in dom_ev)
    dom_us = 1e3 * sum(timer.elapsed_ms(s0, s1) for s0, s1, _ in dom_ev) / dom_launches
    timer.destroy(pool)
    # per-call breakdown (informational): a separate pass after the timed
    # region, every call bracketed by events
    n_ev = len(calls) + 1
    bsteps = min(a.steps, 20)
    pool = timer.create(n_ev * bsteps)
    for k in range(bsteps):
        step(pool[k * n_ev:(k + 1) * n_ev], every_call=True)
    torch.cuda.synchronize()
    kern_us = {k: 1e3 * sum(timer.elapsed_ms(s0, s1) for s0, s1 in v) / len(v)
               for k, v in ev.items()}
    timer.destroy(pool)

    # cold steps (informational): each step alone, bracketed by events, after
    # a 2 GiB read that evicts the 256 MB last-level cache.  (A write flush
    # would leave up to 256 MB of dirty lines whose write-back then lands in
    # the step's first large launch: ~55 us there, measured.)
    flusher = ReadFlush(sa, torch, dev)
    cold = None
    if a.cold_steps > 0:
        cold = cold_steps(timer, stream, calls, names, flusher, a.cold_steps)

    # this device's read ceilings (context for the roofline): the fastest
    # streaming read measured here, and the selected rows read alone
    read_gbps = stream_read_gbps(sa, torch, dev, timer, stream)
    row_read = row_read_gbps(sa, torch, sh, idx, wl, inp, timer, stream, flusher)

    step_bytes = sum(bytes_k.values())
    steps_per_s = 1e3 / ms_per_step
    hbm_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9

    dom_kernel = dict((n, k) for n, _, k in stages)[dom]
    dom_gbps = bytes_k[dom] / (dom_us * 1e-6) / 1e9
    src_hash = _source_hash(KERNEL_SOURCES)
    traffic = measured_traffic(dom_kernel, src_hash)
    roofline = {"bound": "hbm", "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                "traffic": traffic,
                "kernel": "%s (sparse_attn_decode_step_stage, %s)" % (dom_kernel, STAGE_NAMES[
                    dict((n, st) for n, st, _ in stages)[dom]]),
                "bytes_per_launch": bytes_k[dom], "avg_launch_us": round(dom_us, 2),
                "launches_timed": dom_launches, "event_pairs": len(dom_ev),
                "launches_per_event_pair": run, "events_every_steps": period,
                "source_hash": src_hash,
                "read_ceiling_gbps": round(read_gbps, 1),
                "frac_of_read_ceiling": round(dom_gbps / read_gbps, 4),
                "row_read_ceiling_gbps": row_read}

    res = {
        "metric": METRIC, "value": round(steps_per_s, 2), "unit": "steps/s",
        "hbm_gbps": round(hbm_gbps, 1), "hbm_frac": round(hbm_gbps / HBM_PEAK_GBPS, 4),
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4), "gpu_event_ms_per_step": round(gpu_ms / a.steps, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32",
        "storage": "bf16 K/V/q, fp8-e4m3 projected-key cache, int32 indices",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
                   "head_dim": wl.d, "context_N": wl.N, "rank_r": wl.r, "budget_M": wl.M},
        "tokens_per_s": round(steps_per_s * wl.B, 1),
        "step_bytes": step_bytes,
        "plan": PLAN_NAMES.get(plan, str(plan)),
        "kernel_us_breakdown_pass": {k: round(v, 2) for k, v in kern_us.items()},
        "kernel_gbps_breakdown_pass": {k: round(bytes_k[k] / (kern_us[k] * 1e-6) / 1e9, 1)
                                       for k in kern_us
                        if bytes_k[k]},
        "roofline": roofline,
        "cold_step_us": cold,
        "cpu_baseline": None,
        "baselines": None,
    }
    if a.baseline_reps > 0:
        print("bench: comparison baselines", file=sys.stderr, flush=True)
        b = measure_baselines(sa, torch, inp, wl, sh, kp, idx, ws, timer, stream,
                              a.baseline_reps, flusher)
        b["dense_speedup_of_step"] = round(b["dense_attention_us"] / (1e3 * ms_per_step), 2)
        res["baselines"] = b
    if a.cpu_units > 0:
        print("bench: cpu baseline (%d units)" % a.cpu_units, file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inp, wl, a.cpu_units)
    if a.ext_reps > 0:
        print("bench: extensions", file=sys.stderr, flush=True)
        del inp, kp, ws, idx, out
        torch.cuda.empty_cache()
        res["small_workloads"] = measure_small_workloads(sa, torch, dev, timer, stream, flusher,
                                                         max(a.ext_reps, 10))
        res["extensions"] = measure_extensions(sa, torch, dev, a.ext_reps, timer, stream,
                                               flusher)
    else:
        res["extensions"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
