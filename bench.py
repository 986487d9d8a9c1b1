#!/usr/bin/env python3
"""Benchmark of the reduced-precision K/V-cache attention path on one MI355X.

Workload (full context): 48 layers, each 8 kv heads x 32 query heads x head_dim
128 at 262144 cells, batch 1, once with an FP16 cache (1 GiB/layer) and once with
the int8 cache (codes + fp16 scale per 64 dims, 0.516 GiB/layer).  Seeded
synthetic K/V (standard normal, 4 outlier channels x20 per kv head); layer 0 is
filled by kv_append from host-generated values, the other layers are device copies
of it (distinct addresses, so no cache level holds more than a sliver of them).

One step = for each format, for each of the 48 layers: kv_append of one new token
(quantise-on-write or FP16 store) and kv_decode_attn over the cache.  The timed
region holds exactly `--steps` steps between two device synchronisations; the
metric is the decode's algorithmic K/V bytes per step / step time.  The per-call
roofline times the 48 layers' decode calls of one format captured as a HIP graph
(HIP events around each replay on its stream); the same calls launched eagerly with
events around each one are reported beside it.  Side measurements (not in the
step): bulk append rate, the smaller workloads, and the 4096-token prompt chunk at
position 131072 of an int8 cache.

Prints progress to stderr and ONE JSON line to stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn KV read GB/s (% HBM peak) at 262144 ctx, fp16 & int8; append cells/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix, vendor figure
KVH, NQH, HD, CTX, LAYERS = 8, 32, 128, 262144, 48
F16, Q8, K8V4 = 0, 1, 2
BYTES_PER_CELL_HEAD = {F16: 2 * HD * 2, Q8: 2 * (HD + 2 * (HD // 64)),      # K+V per (cell, kv head)
                       K8V4: HD + 2 * (HD // 64) + HD // 2 + 2 * (HD // 32)}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_bytes(fmt, length):
    return length * KVH * BYTES_PER_CELL_HEAD[fmt]


def source_hash(*names):
    """Hash of kernel sources with // comments and blank space dropped, so that a
    comment edit does not invalidate counters taken on the same code."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quantized_kv_cache_q8_amd", "csrc", n)) as f:
            for line in f:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def load_traffic(kernel_key, src_hash):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/), only if the
    kernel source has not changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


# ----------------------------------------------------------------------------
def build_model(kq, torch, seed, cap, warm_len):
    """48 layers x 2 formats, each layer one session (cap cells), layer 0 filled
    with kv_append from seeded host data, layers 1.. device copies."""
    import kvsynth
    log("generating layer K/V on the host")
    xk = kvsynth.kv_tokens(seed, 0, CTX, KVH, HD, "K", outliers=True)
    xv = kvsynth.kv_tokens(seed, 0, CTX, KVH, HD, "V", outliers=True)
    dk = torch.from_numpy(xk[None]).cuda()
    dv = torch.from_numpy(xv[None]).cuda()
    del xk, xv
    model = {}
    append_rate = {}
    for fmt in (F16, Q8):
        sh = kq.make_shape(fmt, KVH, NQH, HD)
        base = kq.Session(fmt, KVH, cap)
        tab0 = kq.session_table([base.entry()])
        lens0 = torch.zeros(1, dtype=torch.int32, device="cuda")
        # bulk append of the whole context, timed (first call warms the code object)
        kq.kv_append(sh, tab0, lens0, 1, 1024, dk[:, :1024].contiguous(), dv[:, :1024].contiguous())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kq.kv_append(sh, tab0, lens0, 1, CTX, dk, dv)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        rw = CTX * KVH * 2 * HD * 4 + kq.kv_cache_bytes(fmt, KVH, CTX, HD, 0) * 2 + \
            kq.kv_cache_bytes(fmt, KVH, CTX, HD, 1) * 2
        append_rate["f16" if fmt == F16 else "int8"] = {
            "cells_per_s": CTX / (ms * 1e-3), "us": ms * 1e3, "GB_s": rw / (ms * 1e-3) / 1e9,
            "frac_hbm": rw / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "cells": CTX,
            "bytes_per_cell": rw // CTX}
        log(f"fmt={fmt}: bulk append {CTX} cells in {ms:.3f} ms")
        layers = [base]
        for i in range(1, LAYERS):
            s = kq.Session(fmt, KVH, cap, fill=None)
            for a, b in zip(s.tensors(), base.tensors()):
                a.copy_(b)
            layers.append(s)
        tabs = [kq.session_table([s.entry()]) for s in layers]
        model[fmt] = dict(shape=sh, layers=layers, tabs=tabs)
        torch.cuda.synchronize()
        log(f"fmt={fmt}: {LAYERS} layers ready")
    del dk, dv
    torch.cuda.empty_cache()
    return model, append_rate


def one_step(kq, torch, model, lens_w, lens_d, q, xk_new, xv_new, ws, out, events=None):
    """One step: for each format and each of the 48 layers, a one-token append at
    lens_w, then a decode over lens_d cells (max_len = the full context, a bound on
    every length); then both lengths advance on the device.  Launches only, so a
    step can be captured as a HIP graph."""
    for fmt, m in model.items():
        sh = m["shape"]
        for li in range(LAYERS):
            tab = m["tabs"][li]
            kq.kv_append(sh, tab, lens_w, 1, 1, xk_new[li], xv_new[li])
            if events is not None:
                e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                e[0].record()
            kq.kv_decode_attn(sh, tab, lens_d, 1, CTX, q[li], 1 / math.sqrt(HD), out, ws[fmt])
            if events is not None:
                e[1].record()
                events[fmt].append(e)
    lens_w += 1
    lens_d += 1


def run_steps(kq, torch, model, n_steps, len0, q, xk_new, xv_new, ws, events=None):
    """n_steps eager steps starting with len0 cached cells; returns the final length."""
    # lens_w: where the new token goes (cells before it); lens_d: cells the decode reads
    lens_w = torch.full((1,), len0, dtype=torch.int32, device="cuda")
    lens_d = torch.full((1,), len0 + 1, dtype=torch.int32, device="cuda")
    out = torch.empty((1, NQH, HD), device="cuda")
    for _ in range(n_steps):
        one_step(kq, torch, model, lens_w, lens_d, q, xk_new, xv_new, ws, out, events)
    return len0 + n_steps


def graph_steps(kq, torch, model, n_warm, n_steps, len0, q, xk_new, xv_new, ws):
    """The same steps with one step captured once as a HIP graph and replayed: n_warm
    untimed replays from len0 cells, then n_steps timed ones (synchronised on both
    sides).  Returns the seconds of the timed replays."""
    lens_w = torch.full((1,), len0, dtype=torch.int32, device="cuda")
    lens_d = torch.full((1,), len0 + 1, dtype=torch.int32, device="cuda")
    out = torch.empty((1, NQH, HD), device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            one_step(kq, torch, model, lens_w, lens_d, q, xk_new, xv_new, ws, out)
    torch.cuda.synchronize()
    assert int(lens_w.item()) == len0          # capturing runs nothing
    for _ in range(n_warm):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_steps):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert int(lens_w.item()) == len0 + n_warm + n_steps
    assert torch.isfinite(out).all().item()
    return t1 - t0


def graph_call_times(kq, torch, model, length, q, ws, reps):
    """Per-call duration of kv_decode_attn as a captured step runs it: for each format,
    the 48 layers' decode calls over `length` cells captured as one HIP graph (no
    appends), replayed `reps` times with HIP events around each replay on the graph's
    stream.  Returns seconds per call (split and merge kernels and the gaps between
    them, without the host's launch cost)."""
    out = torch.empty((1, NQH, HD), device="cuda")
    res = {}
    for fmt, m in model.items():
        lens_d = torch.full((1,), length, dtype=torch.int32, device="cuda")
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                for li in range(LAYERS):
                    kq.kv_decode_attn(m["shape"], m["tabs"][li], lens_d, 1, CTX, q[li],
                                      1 / math.sqrt(HD), out, ws[fmt])
        torch.cuda.synchronize()
        evs = []
        with torch.cuda.stream(stream):
            graph.replay()   # untimed
            for _ in range(reps):
                e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                e[0].record(stream)
                graph.replay()
                e[1].record(stream)
                evs.append(e)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all().item()
        res[fmt] = float(np.mean([a.elapsed_time(b) * 1e-3 for a, b in evs])) / LAYERS
        del graph
    return res


def prefill_side(kq, torch, seed, steps, warmup):
    """4096-token chunk at position 131072 of an int8 cache: compaction and MFMA attention."""
    import kvsynth
    pos0, n_tok = 131072, 4096
    P = pos0 + n_tok
    log("prefill: filling 135168 int8 cells")
    sh = kq.make_shape(Q8, KVH, NQH, HD)
    s = kq.Session(Q8, KVH, P)
    tab = kq.session_table([s.entry()])
    lens = torch.zeros(1, dtype=torch.int32, device="cuda")
    chunk = 32768
    for t0 in range(0, P, chunk):
        n = min(chunk, P - t0)
        xk = kvsynth.kv_tokens(seed, 0, n, KVH, HD, "K", True, sub=1000 + t0)
        xv = kvsynth.kv_tokens(seed, 0, n, KVH, HD, "V", True, sub=1000 + t0)
        lens.fill_(t0)
        kq.kv_append(sh, tab, lens, 1, n, torch.from_numpy(xk[None]).cuda(),
                     torch.from_numpy(xv[None]).cuda())
    q = torch.from_numpy(kvsynth.queries(seed, 0, n_tok, NQH, HD, stream=kvsynth.S_Q_PREFILL)).cuda()
    out = torch.empty((n_tok, NQH, HD), device="cuda")
    ws = torch.empty(kq.kv_prefill_workspace_bytes(sh, P), dtype=torch.uint8, device="cuda")
    half = ws.numel() // 2
    k16 = ws[:half].view(torch.int16)
    v16 = ws[half:].view(torch.int16)
    sm = 1 / math.sqrt(HD)
    for _ in range(warmup):
        kq.kv_prefill_attn(sh, s.entry(), pos0, n_tok, q, sm, out, ws)
    torch.cuda.synchronize()
    ev = []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        kq.kv_compact_f16(sh, s.entry(), P, k16, v16)
        e[1].record()
        kq.kv_prefill_attn(sh, s.entry(), pos0, n_tok, q, sm, out, ws)
        e[2].record()
        ev.append(e)
    torch.cuda.synchronize()
    comp_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    total_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
    attn_ms = max(total_ms - comp_ms, 1e-9)
    pairs = sum(pos0 + i + 1 for i in range(n_tok))
    flop = 4.0 * HD * pairs * NQH
    comp_bytes = P * KVH * (2 * (HD + 4) + 2 * HD * 2)
    assert torch.isfinite(out).all().item()
    return {
        "workload": "int8 cache, 4096-token chunk at position 131072, 8 kv / 32 q heads",
        "tokens_per_s": n_tok / (total_ms * 1e-3), "ms_total": total_ms,
        "compaction_ms": comp_ms, "compaction_GB_s": comp_bytes / (comp_ms * 1e-3) / 1e9,
        "attention_ms": attn_ms, "attention_TFLOP_s": flop / (attn_ms * 1e-3) / 1e12,
        "mfma_frac": flop / (attn_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
        "flop": flop}


CALIB_BYTES = 3 << 28   # 768 MiB: a size no other copy in the probe has


def traffic_probe(kq, torch, seed):
    """Kernels for counter collection (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE): a
    plain device-to-device copy of CALIB_BYTES (the calibration), then per format
    (FP16, int8, K8V4) one 262144-cell layer: bulk append and 3 decodes."""
    import kvsynth
    a = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    xk = torch.from_numpy(kvsynth.kv_tokens(seed, 0, CTX, KVH, HD, "K", True)[None]).cuda()
    xv = torch.from_numpy(kvsynth.kv_tokens(seed, 0, CTX, KVH, HD, "V", True)[None]).cuda()
    q = torch.from_numpy(kvsynth.queries(seed, 0, 1, NQH, HD)).cuda()
    out = torch.empty((1, NQH, HD), device="cuda")
    for fmt in (F16, Q8, K8V4):
        sh = kq.make_shape(fmt, KVH, NQH, HD)
        s = kq.Session(fmt, KVH, CTX)
        tab = kq.session_table([s.entry()])
        lens = torch.zeros(1, dtype=torch.int32, device="cuda")
        kq.kv_append(sh, tab, lens, 1, CTX, xk, xv)
        lens.fill_(CTX)
        ws = kq.kv_decode_workspace(sh, 1, CTX)
        for _ in range(3):
            kq.kv_decode_attn(sh, tab, lens, 1, CTX, q, 1 / math.sqrt(HD), out, ws)
        torch.cuda.synchronize()
        del s
    log("traffic probe done")


def traffic_summary(fetch_dir, write_dir, command):
    """Turn the counter CSVs of two `--traffic-probe` runs (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch) into profiles/hbm_traffic.json.  Each counter is
    scaled by expected / measured on the calibration copy (CALIB_BYTES read and
    written); dispatches of the two runs pair up by dispatch id (same program)."""
    import csv
    import glob

    def load(d, counter):
        rows = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    rows[int(r["Dispatch_Id"])] = (r["Kernel_Name"], float(r["Counter_Value"]))
        if not rows:
            raise SystemExit(f"no {counter} rows under {d}")
        return rows

    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    exp_kib = CALIB_BYTES / 1024
    calib = [i for i, (n, v) in write.items() if "copyBuffer" in n and abs(v - exp_kib) < 0.02 * exp_kib]
    if not calib or any(i not in fetch for i in calib):
        raise SystemExit("calibration copy not found in both runs")
    f_fac = exp_kib / float(np.mean([fetch[i][1] for i in calib]))
    w_fac = exp_kib / float(np.mean([write[i][1] for i in calib]))
    out = {"command": command, "calibration": {
        "kernel": "__amd_rocclr_copyBuffer (device-to-device copy)", "bytes_read": CALIB_BYTES,
        "bytes_written": CALIB_BYTES, "dispatches": len(calib),
        "fetch_KiB": float(np.mean([fetch[i][1] for i in calib])),
        "write_KiB": float(np.mean([write[i][1] for i in calib])),
        "fetch_factor": f_fac, "write_factor": w_fac}}
    ids = sorted(fetch)
    for fmt, key in ((F16, "decode_f16"), (Q8, "decode_int8"), (K8V4, "decode_k8v4")):
        # one kv_decode_attn call = one split kernel (k_decode_split for FP16,
        # k_decode_pair_mv for the int8-K formats at 1, 2 or 4 query heads per kv head,
        # else k_decode_pair) then one k_decode_merge<fmt>
        tags = (f"k_decode_split<{fmt},", f"k_decode_pair<{fmt},", f"k_decode_pair_mv<{fmt},")
        splits = [i for i in ids if any(t in fetch[i][0] for t in tags)]
        per = []
        for i in splits:
            j = i + 1
            assert f"k_decode_merge<{fmt}>" in fetch[j][0], fetch[j][0]
            fk = fetch[i][1] + fetch[j][1]
            wk = write[i][1] + write[j][1]
            per.append((fk, wk, fk * 1024 * f_fac + wk * 1024 * w_fac))
        per = np.array(per)
        out[key] = {"source_hash": source_hash("decode.hip"), "launches": len(per),
                    "context": CTX, "fetch_KiB": float(per[:, 0].mean()),
                    "write_KiB": float(per[:, 1].mean()),
                    "bytes_per_launch": float(per[:, 2].mean()),
                    "algorithmic_bytes_per_launch": decode_bytes(fmt, CTX),
                    "ratio_to_algorithmic": float(per[:, 2].mean()) / decode_bytes(fmt, CTX)}
    for fmt, key in ((F16, "append_f16"), (Q8, "append_int8"), (K8V4, "append_k8v4")):
        a = [i for i in ids if f"k_append<{fmt}>" in fetch[i][0]]
        fk = float(np.mean([fetch[i][1] for i in a]))
        wk = float(np.mean([write[i][1] for i in a]))
        alg = CTX * KVH * 2 * HD * 4 + CTX * KVH * BYTES_PER_CELL_HEAD[fmt]
        out[key] = {"source_hash": source_hash("append.hip"), "cells": CTX, "fetch_KiB": fk,
                    "write_KiB": wk, "bytes_per_launch": fk * 1024 * f_fac + wk * 1024 * w_fac,
                    "algorithmic_bytes_per_launch": alg}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def stream_ceiling(kq, torch, reps=10):
    """Read rate of a plain streaming kernel (kv_probe_stream_read: the decode's
    128-bit non-temporal loads, no arithmetic) over exactly the bytes one decode call
    reads, per format.  Four buffers of that size rotate, so the 256 MB last-level
    cache cannot serve repeats; HIP events on the launch stream around reps x 4
    back-to-back launches, as for the decode."""
    out = {}
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for key, fmt in (("f16", F16), ("int8", Q8)):
        nbytes = decode_bytes(fmt, CTX)
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(4)]
        for b in bufs:
            kq.kv_probe_stream_read(b, sink)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for b in bufs:
                kq.kv_probe_stream_read(b, sink)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * len(bufs))
        out[key] = {"bytes": nbytes, "us": us, "GB_s": nbytes / us / 1e3}
        del bufs
        torch.cuda.empty_cache()
    return out


def _time_calls(torch, calls, reps):
    """Mean HIP-event time (s) of each of the zero-argument callables in calls,
    recorded around it on the launch stream over reps rounds."""
    ev = [[] for _ in calls]
    for _ in range(reps):
        for i, f in enumerate(calls):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            ev[i].append((e0, e1))
    torch.cuda.synchronize()
    return [float(np.mean([a.elapsed_time(b) for a, b in e])) * 1e-3 for e in ev]


def _warm(torch, calls, ms=30.0):
    """Untimed rounds of the callables until ms of wall time have passed: the clocks
    settle at the load's level (a phase that left the GPU mostly idle, such as the
    host-link copies before it, otherwise costs the first timed rounds several %)."""
    t0 = time.perf_counter()
    while True:
        for f in calls:
            f()
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            return


def _time_loop(torch, calls, reps):
    """Mean seconds per call of the callables in calls run back to back, reps rounds,
    with one pair of HIP events around the whole run (no per-call events between
    launches)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        for f in calls:
            f()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (reps * len(calls))


def _time_graph(torch, calls, reps):
    """Mean seconds per call of the callables in calls, in order, repeated to at least
    32 calls and captured once as a HIP graph, replayed reps times (HIP events around
    each replay on the graph's stream): the calls as a captured step runs them, without
    the host's launches (the repetition spreads the graph's own launch over many calls)."""
    calls = list(calls) * max(1, 32 // len(calls))
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for f in calls:
                f()
    torch.cuda.synchronize()
    evs = []
    with torch.cuda.stream(stream):
        graph.replay()   # untimed
        for _ in range(reps):
            e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            e[0].record(stream)
            graph.replay()
            e[1].record(stream)
            evs.append(e)
    torch.cuda.synchronize()
    del graph
    return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e-3 / len(calls)


def _stream_us(kq, torch, nbytes, reps=10):
    """Microseconds per kv_probe_stream_read over nbytes, four buffers in turn."""
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(4)]
    calls = [lambda b=b: kq.kv_probe_stream_read(b, sink) for b in bufs]
    for f in calls:
        f()
    t = _time_loop(torch, calls, reps)
    del bufs
    torch.cuda.empty_cache()
    return t * 1e6


def side_configs(kq, torch, steps=10, warmup=3):
    """The smaller workloads: the 64-session int8 batch (session lengths uniform on
    [1024, 65536], one session table; a step is one batched 1-token append and one
    batched decode), and single-session decodes at 32768 cells (F16) and 131072
    cells (int8) over 4 layer copies in turn, so the 256 MB last-level cache cannot
    serve repeats.  Cache contents come from seeded host K/V (outlier channels)."""
    import kvsynth
    out = {}
    sm = 1 / math.sqrt(HD)

    # ---- 64 sessions ---------------------------------------------------------
    w = kvsynth.WORKLOADS["batched64_q8"]
    lens = [int(x) for x in kvsynth.session_lengths(w["seed"], w["batch"], w["lo"], w["hi"])]
    n_sess, hi = len(lens), max(lens)
    sh = kq.make_shape(Q8, KVH, NQH, HD)
    dk = torch.from_numpy(kvsynth.kv_tokens(w["seed"], 0, hi, KVH, HD, "K", True)[None]).cuda()
    dv = torch.from_numpy(kvsynth.kv_tokens(w["seed"], 0, hi, KVH, HD, "V", True)[None]).cuda()
    sess = [kq.Session(Q8, KVH, kvsynth.round_up(n + steps + warmup + 1, 64)) for n in lens]
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    for s_, n in zip(sess, lens):
        kq.kv_append(sh, kq.session_table([s_.entry()]), zero, 1, n,
                     dk[:, :n].contiguous(), dv[:, :n].contiguous())
    del dk, dv
    tab = kq.session_table([s_.entry() for s_ in sess])
    lens_w = torch.tensor(lens, dtype=torch.int32, device="cuda")
    lens_d = lens_w + 1
    q = torch.from_numpy(kvsynth.queries(w["seed"], 0, n_sess, NQH, HD)).cuda()
    xk1 = torch.from_numpy(kvsynth.kv_tokens(w["seed"], 0, n_sess, KVH, HD, "K", True,
                                             stream=kvsynth.S_K_NEW)[:, None]).cuda()
    xv1 = torch.from_numpy(kvsynth.kv_tokens(w["seed"], 0, n_sess, KVH, HD, "V", True,
                                             stream=kvsynth.S_V_NEW)[:, None]).cuda()
    max_len = hi + steps + warmup + 1
    ws = kq.kv_decode_workspace(sh, n_sess, max_len)
    o = torch.empty((n_sess, NQH, HD), device="cuda")
    t_app, t_dec, read = [], [], 0
    for step in range(warmup + steps):
        ta, td = _time_calls(torch, [
            lambda: kq.kv_append(sh, tab, lens_w, n_sess, 1, xk1, xv1),
            lambda: kq.kv_decode_attn(sh, tab, lens_d, n_sess, max_len, q, sm, o, ws)], 1)
        if step >= warmup:
            t_app.append(ta)
            t_dec.append(td)
            read += decode_bytes(Q8, int(lens_d.sum().item()))
        lens_w += 1
        lens_d += 1
    assert torch.isfinite(o).all().item()
    # the batched decode alone as a captured step runs it (lengths as they ended)
    t_g = _time_graph(torch, [lambda: kq.kv_decode_attn(sh, tab, lens_d, n_sess, max_len, q, sm,
                                                        o, ws)], steps)
    read_g = decode_bytes(Q8, int(lens_d.sum().item()))
    out["batched64_int8"] = {
        "workload": "64 int8 sessions, lengths uniform on [1024, 65536] (sum "
                    f"{sum(lens)}), one session table; a step = batched 1-token append + "
                    "batched decode",
        "decode_us": float(np.mean(t_dec)) * 1e6,
        "decode_GB_s": read / sum(t_dec) / 1e9,
        "decode_frac_hbm": read / sum(t_dec) / 1e9 / HBM_PEAK_GBS,
        "decode_us_graph": t_g * 1e6,
        "decode_frac_hbm_graph": read_g / t_g / 1e9 / HBM_PEAK_GBS,
        "append_us": float(np.mean(t_app)) * 1e6,
        "append_cells_per_s": n_sess / float(np.mean(t_app))}
    log(f"batched64 int8: decode {out['batched64_int8']['decode_us']:.1f} us = "
        f"{out['batched64_int8']['decode_GB_s']:.0f} GB/s; append "
        f"{out['batched64_int8']['append_us']:.1f} us per 64 cells")
    del sess, tab, ws
    torch.cuda.empty_cache()

    # ---- single sessions at 32768 (F16) and 131072 (int8) cells, and the K8V4 ---
    # ---- format at the full 262144 cells ----------------------------------------
    for key, fmt in (("f16_ctx32768", F16), ("q8_ctx131072", Q8), ("k8v4_ctx262144", K8V4)):
        w = kvsynth.WORKLOADS[key] if key in kvsynth.WORKLOADS else \
            dict(kvsynth.WORKLOADS["full_ctx262144_48l"], fmt="k8v4")
        ctx = w["ctx"]
        sh = kq.make_shape(fmt, KVH, NQH, HD)
        dk = torch.from_numpy(kvsynth.kv_tokens(w["seed"], 0, ctx, KVH, HD, "K", True)[None]).cuda()
        dv = torch.from_numpy(kvsynth.kv_tokens(w["seed"], 0, ctx, KVH, HD, "V", True)[None]).cuda()
        cap = kvsynth.round_up(ctx, 64)
        copies = []
        app = None
        for i in range(4):
            s_ = kq.Session(fmt, KVH, cap)
            if i == 1:   # the second fill is timed (the first warms the code)
                app = _time_calls(torch, [lambda: kq.kv_append(
                    sh, kq.session_table([s_.entry()]), zero, 1, ctx, dk, dv)], 1)[0]
            else:
                kq.kv_append(sh, kq.session_table([s_.entry()]), zero, 1, ctx, dk, dv)
            copies.append(s_)
        del dk, dv
        tabs = [kq.session_table([s_.entry()]) for s_ in copies]
        ld = torch.full((1,), ctx, dtype=torch.int32, device="cuda")
        q = torch.from_numpy(kvsynth.queries(w["seed"], 0, 1, NQH, HD)).cuda()
        ws = kq.kv_decode_workspace(sh, 1, ctx)
        o = torch.empty((1, NQH, HD), device="cuda")
        calls = [lambda t=t: kq.kv_decode_attn(sh, t, ld, 1, ctx, q, sm, o, ws) for t in tabs]
        _warm(torch, calls)
        # back to back over the 4 copies (as a model's layers run): the rate; and with
        # events around each call, which adds each launch's gap
        t = _time_loop(torch, calls, steps)
        t_each = float(np.mean(_time_calls(torch, calls, steps)))
        t_graph = _time_graph(torch, calls, steps)
        nb = decode_bytes(fmt, ctx)
        name = {F16: "F16", Q8: "int8", K8V4: "K8V4 (int8 K, rotated 4-bit V)"}[fmt]
        out[key] = {"workload": f"{name} cache, {ctx} cells, 4 copies in turn, back to back",
                    "decode_us": t * 1e6, "decode_bytes": nb,
                    "decode_GB_s": nb / t / 1e9, "decode_frac_hbm": nb / t / 1e9 / HBM_PEAK_GBS,
                    "decode_us_events_each": t_each * 1e6,
                    "decode_us_graph": t_graph * 1e6,
                    "decode_frac_hbm_graph": nb / t_graph / 1e9 / HBM_PEAK_GBS,
                    "bulk_append_cells_per_s": ctx / app}
        # the same copy every call: a layer that fits the 256 MB last-level cache stays
        # in it (what one layer decoded in a loop would see); rotated above is the rate
        hot = [lambda: kq.kv_decode_attn(sh, tabs[0], ld, 1, ctx, q, sm, o, ws)]
        _warm(torch, hot)
        th = _time_loop(torch, hot, 4 * steps)
        out[key]["hot_decode_us"] = th * 1e6
        out[key]["hot_decode_GB_s"] = nb / th / 1e9
        # a decode step's one-token append (quantise-on-write for int8), per call
        ld1 = torch.full((1,), ctx - 1, dtype=torch.int32, device="cuda")
        x1k = torch.from_numpy(kvsynth.kv_tokens(w["seed"], 0, 1, KVH, HD, "K", True,
                                                 stream=kvsynth.S_K_NEW)[None]).cuda()
        x1v = torch.from_numpy(kvsynth.kv_tokens(w["seed"], 0, 1, KVH, HD, "V", True,
                                                 stream=kvsynth.S_V_NEW)[None]).cuda()
        app1 = [lambda t=t: kq.kv_append(sh, t, ld1, 1, 1, x1k, x1v) for t in tabs]
        _warm(torch, app1, 10.0)
        out[key]["step_append_us"] = _time_loop(torch, app1, steps) * 1e6
        log(f"{key}: decode {t * 1e6:.1f} us = {nb / t / 1e9:.0f} GB/s (graph {t_graph * 1e6:.1f} us, "
            f"hot {th * 1e6:.1f} us); one-token append {out[key]['step_append_us']:.1f} us")
        if fmt == Q8:
            out["row_moves_int8"] = row_moves(kq, torch, sh, copies[0], copies[1], ctx)
        del copies, tabs, ws
        torch.cuda.empty_cache()
        # a plain streaming read of the same bytes (four buffers in turn, back to back)
        out[key]["stream_ceiling_us"] = _stream_us(kq, torch, nb, steps)
        out[key]["vs_stream_ceiling"] = out[key]["stream_ceiling_us"] / (t * 1e6)
    out.update(paged_and_streamed(kq, torch, steps, warmup))
    return out


def paged_and_streamed(kq, torch, steps, warmup):
    """Paged sessions and the streamed window.

    paged_int8_ctx262144, paged_f16_ctx262144: the full 262144-cell single-session
    decode read through a
    page table: identity pages over the session itself, and a pool whose 4096 pages of
    64 cells sit at a seeded random permutation of its slots; set against the
    contiguous decode of the same cache (two caches in turn, each larger than the
    last-level cache).

    streamed_int8_ctx32768: 4 sessions of 32768 cells in pinned host stores and a
    1024-slot window (two sessions' worth).  Visiting them in the order 0,1,2,3,...
    misses every page (each map copies a whole session over the host link); visiting
    0,1,0,1,... hits every page after the first pass.  A step is kv_window_map + the
    paged decode, timed by the host clock around the step and a synchronize."""
    import kvsynth
    out = {}
    sm = 1 / math.sqrt(HD)
    seed = kvsynth.WORKLOADS["full_ctx262144_48l"]["seed"]
    sh = kq.make_shape(Q8, KVH, NQH, HD)
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")

    # ---- paged decode at the full context, int8 and F16 -------------------------
    ctx, P = CTX, kq.KV_PAGE_ROWS
    npg = ctx // P
    for fmt, key, name in ((Q8, "paged_int8_ctx262144", "int8"), (F16, "paged_f16_ctx262144", "F16")):
        shf = kq.make_shape(fmt, KVH, NQH, HD)
        dk = torch.from_numpy(kvsynth.kv_tokens(seed, 0, ctx, KVH, HD, "K", True)[None]).cuda()
        dv = torch.from_numpy(kvsynth.kv_tokens(seed, 0, ctx, KVH, HD, "V", True)[None]).cuda()
        a = kq.Session(fmt, KVH, ctx)
        kq.kv_append(shf, kq.session_table([a.entry()]), zero, 1, ctx, dk, dv)
        del dk, dv
        perm = torch.from_numpy(np.random.default_rng(seed).permutation(npg).astype(np.int32)).cuda()
        b = kq.Session(fmt, KVH, ctx)
        for ta, tb in zip(a.tensors(), b.tensors()):   # page p of a -> slot perm[p] of b
            tb.view(KVH, npg, -1)[:, perm.long()] = ta.view(KVH, npg, -1)
        ident = torch.arange(npg, dtype=torch.int32, device="cuda")
        tab_a, tab_b = kq.session_table([a.entry()]), kq.session_table([b.entry()])
        ld = torch.full((1,), ctx, dtype=torch.int32, device="cuda")
        q = torch.from_numpy(kvsynth.queries(seed, 0, 1, NQH, HD)).cuda()
        ws = kq.kv_decode_workspace(shf, 1, ctx)
        o = [torch.empty((1, NQH, HD), device="cuda") for _ in range(3)]
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        calls = [lambda: kq.kv_decode_attn(shf, tab_a, ld, 1, ctx, q, sm, o[0], ws),
                 lambda: kq.kv_decode_attn_paged(shf, tab_b, perm, npg, ld, 1, ctx, q, sm, o[1],
                                                 ws, st),
                 lambda: kq.kv_decode_attn_paged(shf, tab_a, ident, npg, ld, 1, ctx, q, sm, o[2],
                                                 ws, st),
                 lambda: kq.kv_decode_attn_paged(shf, tab_b, perm, npg, ld, 1, ctx, q, sm, o[1],
                                                 ws, st)]
        _warm(torch, calls)
        t = _time_calls(torch, calls, steps)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert torch.equal(o[0], o[1]) and torch.equal(o[0], o[2]), "paged decode differs"
        nb = decode_bytes(fmt, ctx)
        t_res, t_perm, t_id = t[0], (t[1] + t[3]) / 2, t[2]
        out[key] = {
            "workload": f"{name} cache, 262144 cells, 4096 pages of 64 cells; two caches in turn",
            "resident_us": t_res * 1e6, "paged_identity_us": t_id * 1e6,
            "paged_permuted_us": t_perm * 1e6, "decode_bytes": nb,
            "paged_permuted_GB_s": nb / t_perm / 1e9,
            "paged_permuted_frac_hbm": nb / t_perm / 1e9 / HBM_PEAK_GBS,
            "paging_overhead": t_perm / t_res - 1.0,
            "outputs_bitwise_equal": True}
        log(f"paged {name} 262144: resident {t_res * 1e6:.1f} us, identity pages {t_id * 1e6:.1f} us, "
            f"permuted pages {t_perm * 1e6:.1f} us ({nb / t_perm / 1e9:.0f} GB/s)")
        del a, b, tab_a, tab_b, ws, perm, ident
        torch.cuda.empty_cache()

    # ---- streamed window ------------------------------------------------------
    n, n_st, n_slots = 32768, 4, 1024
    npg = n // P
    stores, host_pages = [], []
    for s in range(n_st):
        xk = torch.from_numpy(kvsynth.kv_tokens(seed + 1 + s, 0, n, KVH, HD, "K", True)[None])
        xv = torch.from_numpy(kvsynth.kv_tokens(seed + 1 + s, 0, n, KVH, HD, "V", True)[None])
        tmp = kq.Session(Q8, KVH, n)
        kq.kv_append(sh, kq.session_table([tmp.entry()]), zero, 1, n, xk.cuda(), xv.cuda())
        hs = kq.Session(Q8, KVH, n, pinned=True)
        for ta, tb in zip(tmp.tensors(), hs.tensors()):
            tb.copy_(ta.cpu())
        stores.append(hs)
        host_pages.append(torch.full((npg,), -1, dtype=torch.int32).pin_memory())
    del tmp
    pool = kq.Session(Q8, KVH, n_slots * P)
    tab = kq.session_table([pool.entry()])
    d_pages = torch.zeros(npg, dtype=torch.int32, device="cuda")
    ld = torch.full((1,), n, dtype=torch.int32, device="cuda")
    ws = kq.kv_decode_workspace(sh, 1, n)
    y = torch.empty((1, NQH, HD), device="cuda")
    row_bytes = kq.kv_rows_bytes(sh, P)

    def run(order):
        win = kq.Window(n_slots)
        for hp in host_pages:
            hp.fill_(-1)
        ts, copied = [], []
        for i, s in enumerate(order):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            c = win.map(sh, stores[s], s, npg, pool, host_pages[s], d_pages)
            kq.kv_decode_attn_paged(sh, tab, d_pages, npg, ld, 1, n, q, sm, y, ws, st)
            torch.cuda.synchronize()
            if i >= 2 * n_st:
                ts.append(time.perf_counter() - t0)
                copied.append(c)
        return float(np.mean(ts)), float(np.mean(copied))

    reps = 2 * n_st + max(steps, 8)
    t_miss, c_miss = run([i % n_st for i in range(reps)])
    t_hit, c_hit = run([i % 2 for i in range(reps)])
    assert int(st.item()) == 0
    miss_bytes = c_miss * row_bytes
    out["streamed_int8_ctx32768"] = {
        "workload": "4 int8 sessions of 32768 cells in pinned host stores, a 1024-slot "
                    "window (2 sessions); a step = kv_window_map + paged decode, host clock",
        "miss_step_us": t_miss * 1e6, "miss_pages_per_step": c_miss,
        "miss_host_to_device_GB_s": miss_bytes / t_miss / 1e9,
        "hit_step_us": t_hit * 1e6, "hit_pages_per_step": c_hit}
    log(f"streamed int8 32768: all-miss step {t_miss * 1e6:.0f} us ({c_miss:.0f} pages, "
        f"{miss_bytes / t_miss / 1e9:.1f} GB/s), all-hit step {t_hit * 1e6:.1f} us")
    return out


def row_moves(kq, torch, sh, src, dst, n, reps=5):
    """Moving all n rows of one int8 layer (every array, codes and scales): a device
    copy into another session, a gather into pinned host memory and the scatter back,
    and a saved image of the session (header and token ids written by the host, body
    and scales copied) built and loaded back; HIP events on the launch stream, bytes
    moved (the image's whole size for the image calls) per second."""
    nbytes = kq.kv_rows_bytes(sh, n)
    host = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    ibytes = kq.kv_image_bytes(sh, n)
    image = torch.empty(ibytes, dtype=torch.uint8).pin_memory()
    tokens = torch.arange(n, dtype=torch.int32)
    calls = [lambda: kq.kv_copy_rows(sh, src.entry(), 0, dst.entry(), 0, n),
             lambda: kq.kv_gather_rows(sh, src.entry(), 0, n, host),
             lambda: kq.kv_scatter_rows(sh, dst.entry(), 0, n, host),
             lambda: kq.kv_image_save(sh, src.entry(), n, tokens, image),
             lambda: kq.kv_image_load(sh, dst.entry(), image)]
    _time_calls(torch, calls, 1)
    t = _time_calls(torch, calls, reps)
    res = {"rows": n, "bytes": nbytes, "image_bytes": ibytes}
    names = ("device_copy", "gather_to_pinned_host", "scatter_from_pinned_host",
             "image_save_to_pinned_host", "image_load_from_pinned_host")
    for name, ti, b in zip(names, t, (nbytes,) * 3 + (ibytes,) * 2):
        res[name] = {"us": ti * 1e6, "GB_s": b / ti / 1e9}
    log("row moves int8: " + ", ".join(f"{k} {v['GB_s']:.0f} GB/s" for k, v in res.items()
                                        if isinstance(v, dict)))
    return res


def cpu_prefill_sample(cache, seed, n_rows=64):
    """The oracle's prompt-chunk attention at the prefill workload's shape (4096-token
    chunk at position 131072, P = 135168, 32 query heads) on n_rows evenly spaced
    rows of the chunk, over the given int8 cache's compacted copy; the full chunk's
    time is extrapolated by its share of the causal flops."""
    import kvsynth
    import oracle
    pos0, n_tok = 131072, 4096
    P = pos0 + n_tok
    q = kvsynth.queries(seed, 0, n_tok, NQH, HD, stream=kvsynth.S_Q_PREFILL)
    rows = np.linspace(0, n_tok - 1, n_rows).round().astype(np.int64)
    t0 = time.perf_counter()
    k16, v16 = oracle.compact_f16(cache, P)
    t1 = time.perf_counter()
    oracle.prefill_attn(q, k16, v16, pos0, 1 / math.sqrt(HD), rows=rows)
    t2 = time.perf_counter()
    flop_rows = 4.0 * HD * NQH * float(np.sum(pos0 + rows + 1))
    flop_all = 4.0 * HD * NQH * float(np.sum(pos0 + np.arange(n_tok) + 1))
    return {"rows": n_rows, "attention_s": t2 - t1, "GFLOP_s": flop_rows / (t2 - t1) / 1e9,
            "compaction_s": t1 - t0,
            "extrapolated_chunk_s": (t2 - t1) * flop_all / flop_rows + (t1 - t0),
            "note": "extrapolated from the sampled rows by causal flops"}


def cpu_baseline_leg(seed, repeats=4):
    """The oracle, as it stands, on a bounded sample of the workload: one of the 48
    layers (8 kv heads, 32 query heads, 262144 cells), both formats: cache write
    of every cell, then the fp64 decode (repeated)."""
    import kvsynth
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    xk = kvsynth.kv_tokens(seed, 0, CTX, KVH, HD, "K", outliers=True)
    xv = kvsynth.kv_tokens(seed, 0, CTX, KVH, HD, "V", outliers=True)
    q = kvsynth.queries(seed, 0, 1, NQH, HD)[0]
    res = {}
    total_bytes, total_s = 0, 0.0
    for fmt in (F16, Q8):
        t0 = time.perf_counter()
        c = oracle.Cache(fmt, KVH, CTX, HD)
        c.append(0, xk, xv)
        t1 = time.perf_counter()
        for _ in range(repeats):
            K = c.dequant("k", CTX)
            V = c.dequant("v", CTX)
            oracle.decode_attn(q, K, V, CTX, 1 / math.sqrt(HD))
            del K, V
        t2 = time.perf_counter()
        nbytes = decode_bytes(fmt, CTX) * repeats
        # the same decode with BLAS held to one thread: the per-core rate
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                t3 = time.perf_counter()
                K = c.dequant("k", CTX)
                V = c.dequant("v", CTX)
                oracle.decode_attn(q, K, V, CTX, 1 / math.sqrt(HD))
                del K, V
                t4 = time.perf_counter()
            one = decode_bytes(fmt, CTX) / (t4 - t3) / 1e9
        except Exception:  # pragma: no cover
            one = None
        res["f16" if fmt == F16 else "int8"] = {
            "decode_GB_s": nbytes / (t2 - t1) / 1e9, "decode_s": (t2 - t1) / repeats,
            "decode_GB_s_one_thread": one,
            "append_cells_per_s": CTX / (t1 - t0), "append_s": t1 - t0}
        total_bytes += nbytes
        total_s += t2 - t1
        if fmt == Q8:
            res["prefill"] = cpu_prefill_sample(c, seed)
        del c
    cores = len(os.sched_getaffinity(0))
    return {"value": total_bytes / total_s / 1e9, "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"one layer of the workload (8 kv heads, 32 query heads, 262144 cells), "
                      f"FP16 and int8: oracle cache write of every cell, then its fp64 decode "
                      f"{repeats}x; value = decode K/V bytes / decode time (per_format.int8."
                      f"prefill: the oracle's prompt-chunk attention on 64 sampled rows of the "
                      f"4096-token chunk at 131072, extrapolated); numpy elementwise "
                      f"work on 1 thread, BLAS on {blas_threads} of {cores} cores",
            "host_cores": cores, "per_format": res}


# ----------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=44)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-side-configs", action="store_true",
                    help="skip the smaller workloads (batch, short contexts, K8V4)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the prompt-chunk side (compaction + attention, 2 timed "
                         "calls), e.g. under rocprofv3 counters")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run only what the HBM-traffic counters are read on: a 768 MiB device "
                         "copy (calibration), then per format one 262144-cell layer: bulk "
                         "append and 3 decodes")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="(no GPU) write profiles/hbm_traffic.json from the rocprofv3 counter "
                         "output of two --traffic-probe runs")
    ap.add_argument("--traffic-command", default="",
                    help="with --traffic-summary: the rocprofv3 commands, recorded in the file")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, args.traffic_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode (--gpus {args.gpus} "
              "requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import quantized_kv_cache_q8_amd as kq

    if args.traffic_probe:
        traffic_probe(kq, torch, args.seed)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_side(kq, torch, 55, steps=2, warmup=1)}), flush=True)
        return

    n_steps, n_warm = args.steps, args.warmup
    cap = ((CTX + 63) // 64) * 64
    len0 = CTX - (n_steps + n_warm)          # the last step decodes over exactly 262144 cells
    model, append_rate = build_model(kq, torch, args.seed, cap, len0)

    import kvsynth
    q = [torch.from_numpy(kvsynth.queries(args.seed, li, 1, NQH, HD)).cuda() for li in range(LAYERS)]
    xk_new = [torch.from_numpy(kvsynth.kv_tokens(args.seed, li, 1, KVH, HD, "K", True,
                                                 stream=kvsynth.S_K_NEW)[None]).cuda()
              for li in range(LAYERS)]
    xv_new = [torch.from_numpy(kvsynth.kv_tokens(args.seed, li, 1, KVH, HD, "V", True,
                                                 stream=kvsynth.S_V_NEW)[None]).cuda()
              for li in range(LAYERS)]
    ws = {fmt: kq.kv_decode_workspace(model[fmt]["shape"], 1, CTX) for fmt in model}

    log(f"warmup {n_warm} eager steps")
    length = run_steps(kq, torch, model, n_warm, len0, q, xk_new, xv_new, ws)
    torch.cuda.synchronize()
    bytes_total = sum(decode_bytes(fmt, length + s + 1) * LAYERS for fmt in (F16, Q8)
                      for s in range(n_steps))
    # one step captured as a HIP graph and replayed from len0 again (the appends rewrite
    # the same cells): n_warm untimed replays, then the n_steps timed ones -- the value
    log(f"graph: warmup {n_warm}, timing {n_steps} replays")
    g_s = graph_steps(kq, torch, model, n_warm, n_steps, len0, q, xk_new, xv_new, ws)
    step_s = g_s / n_steps
    value = bytes_total / g_s / 1e9
    log(f"graph steps: {step_s * 1e3:.2f} ms per step, {value:.0f} GB/s")
    # the same n_steps again, launched eagerly with HIP events around every decode call
    # (the per-call rooflines), at the clocks the graph steps ran at
    log(f"eager: timing {n_steps} steps, events around each decode")
    events = {F16: [], Q8: []}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    end_len = run_steps(kq, torch, model, n_steps, length, q, xk_new, xv_new, ws, events)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert end_len == CTX
    eager_step_s = (t1 - t0) / n_steps
    eager_value = bytes_total / (t1 - t0) / 1e9
    log(f"eager steps: {eager_step_s * 1e3:.2f} ms per step, {eager_value:.0f} GB/s")

    # the decode calls alone, as a captured step runs them (over the full context)
    log("graph of the 48 decode calls per format: per-call durations")
    g_call = graph_call_times(kq, torch, model, CTX, q, ws, reps=n_steps)

    roof = {}
    for fmt in (F16, Q8):
        durs = [a.elapsed_time(b) * 1e-3 for a, b in events[fmt]]
        avg_eager = float(np.mean(durs))
        avg = g_call[fmt]
        per_launch = float(decode_bytes(fmt, CTX))
        ach = per_launch / avg / 1e9
        key = "decode_f16" if fmt == F16 else "decode_int8"
        roof[fmt] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS,
                     "traffic": load_traffic(key, source_hash("decode.hip")),
                     "kernel": ("k_decode_split" if fmt == F16 else "k_decode_pair_mv") +
                               " + k_decode_merge (one kv_decode_attn call)",
                     "avg_us": avg * 1e6, "algorithmic_bytes_per_launch": per_launch,
                     "timing": "HIP events around replays of a HIP graph of the 48 layers' "
                               "decode calls over 262144 cells (the launch form of the step), "
                               "per call",
                     "avg_us_eager_events": avg_eager * 1e6,
                     "achieved_eager_events": float(np.mean(
                         [decode_bytes(fmt, length + s + 1) for s in range(n_steps)])) /
                         avg_eager / 1e9,
                     "tokens_per_s_48_layers": 1.0 / (avg * LAYERS)}
        if fmt == Q8:
            roof[fmt]["note"] = ("both products on the matrix cores (K logits as int8, the V "
                                 "sums as bf16 with fp32 accumulation); the kernel is bound by "
                                 "the HBM stream")
        log(f"fmt={fmt}: {avg * 1e6:.1f} us per call in the graph ({ach:.0f} GB/s, "
            f"{ach / HBM_PEAK_GBS:.1%}); {avg_eager * 1e6:.1f} us by events around eager calls")
    dominant = F16 if roof[F16]["avg_us"] >= roof[Q8]["avg_us"] else Q8
    del model
    torch.cuda.empty_cache()

    ceiling = stream_ceiling(kq, torch)
    for fmt, key in ((F16, "f16"), (Q8, "int8")):
        roof[fmt]["vs_stream_ceiling"] = roof[fmt]["achieved"] / ceiling[key]["GB_s"]
        log(f"stream ceiling {key}: {ceiling[key]['GB_s']:.0f} GB/s over {ceiling[key]['bytes']} B; "
            f"decode at {roof[fmt]['vs_stream_ceiling']:.1%} of it")

    sides = None if args.no_side_configs else side_configs(kq, torch)

    prefill = None
    if not args.no_prefill:
        prefill = prefill_side(kq, torch, 55, steps=5, warmup=1)
        log(f"prefill: {prefill['attention_ms']:.2f} ms attention, "
            f"{prefill['attention_TFLOP_s']:.0f} TFLOP/s ({prefill['mfma_frac']:.1%})")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline_leg(args.seed)

    line = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": n_steps,
        "warmup": n_warm, "ms_per_step": step_s * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "full-context decode: 48 layers x (8 kv heads, 32 query heads, "
                               "head_dim 128), 262144 cells, batch 1, FP16 cache and int8 cache; "
                               "a step appends one token per layer and decodes, both formats",
                   "layers": LAYERS, "kv_heads": KVH, "q_heads": NQH, "head_dim": HD,
                   "context": CTX, "batch": 1, "formats": ["f16", "int8"],
                   "launch": "one step captured as a HIP graph, replayed per step"},
        "eager": {"value": eager_value, "ms_per_step": eager_step_s * 1e3},
        "frac_hbm": value / HBM_PEAK_GBS,
        "roofline": roof[dominant],
        "roofline_int8" if dominant == F16 else "roofline_f16": roof[Q8 if dominant == F16 else F16],
        "cpu_baseline": cpu,
        "append_bulk": append_rate,
        "stream_ceiling": ceiling,
        "side_configs": sides,
        "prefill": prefill,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
