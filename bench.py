#!/usr/bin/env python3
"""Benchmark of the verify-attention hot path on one MI355X.

A step is one pass of the whole path over one batch: roll back the previous
step's draft rows (host, O(1) per sequence), append the new rows into their
blocks and run the verify attention over them (kv_append_verify: for the
plain formats the attention kernel writes the rows itself; compressed caches
quantize on append in a launch before it), partials + merge.  --separate
times kv_append + spec_verify_attn instead.  Steps rotate over enough independent layer
caches (>= 1 GiB in all) that the 256 MB Infinity Cache cannot hold the
working set, as successive layers of a model would.

Reported: verified query-tokens/s (the metric's first half) as ``value``,
effective KV GB/s and % of HBM peak, the attention kernel's roofline (its
algorithmic bytes over its average duration, timed live with HIP events on
the launch stream), and the fp64 CPU oracle timed on a bounded sample.

With no --workload the line's value is the compressed (TQ3) cache at 100K
context, 4 sequences, and the bf16 cache of the same shape is reported
beside it under "also"; a streaming-read probe gives the practical read
ceiling both are also compared with.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

EVENT_STRIDE = 7  # timed steps per HIP-event sample (see event_stride)
METRIC = "verified query-tokens/s + effective KV GB/s (% HBM peak), spec-verify attention"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
ATTN_SRC = os.path.join(ROOT, "speculative_verify_attention_amd", "csrc", "attn.hip")


def workloads():
    from speculative_verify_attention_amd import synth

    return {
        "tiny": lambda: (synth.tiny(), None),
        "qwen3_4b_dense": lambda: (synth.qwen3_4b_dense(), None),
        "gemma_interleaved": lambda: (synth.gemma_interleaved(), [(512, 50.0), (0, 50.0)]),
        "gemma_tq3": lambda: (synth.gemma_interleaved(fmt=synth.KV_TQ3), [(512, 50.0), (0, 50.0)]),
        "tq3_512": lambda: (synth.tq3_long(512), None),
        "tq3_40000": lambda: (synth.tq3_long(40000), None),
        "tq3_100000": lambda: (synth.tq3_long(100000), None),
        "bf16_100000": lambda: (synth.tq3_long(100000, fmt=synth.KV_BF16), None),
        "mixed_batch": lambda: (synth.mixed_batch(), None),
    }


# The acceptance step after the verify forward (not part of the default run):
# 16 sequences with 4 drafts each, a Qwen3-sized vocabulary, draft-model
# logits, temperature 0.8.
ACCEPT_WORKLOADS = {
    "accept_qwen3_sampled": dict(n_draft=[4] * 16, vocab=151936, temperature=0.8, with_draft=True),
    "accept_qwen3_greedy": dict(n_draft=[4] * 16, vocab=151936, temperature=0.0, with_draft=True),
}


def event_stride(steps):
    """Timed steps per HIP-event sample.  A pair of events around a launch
    adds ~5 us of GPU time to its step (measured on the dense workload: 66.1
    us per step with events on every step, 60.5 us with none), so the events
    bracket the attention launch of every EVENT_STRIDE-th timed step only
    (of fewer steps, every k-th with k chosen for at least five samples); the
    step rate counts every step."""
    return max(1, min(EVENT_STRIDE, steps // 5))


def percentiles(ms):
    """Nearest-rank p10, p50 and p90 of per-call durations (ms)."""
    ks = sorted(ms)
    return [round(ks[min(len(ks) - 1, max(0, math.ceil(f * len(ks)) - 1))], 5) for f in (0.1, 0.5, 0.9)]


def run_accept(args, name):
    """Times spec_accept on seeded logits resident in HBM (replicated past
    1 GiB so that every call reads HBM, not the MALL)."""
    import time

    import torch

    from speculative_verify_attention_amd import spec_accept, spec_accept_workspace_bytes, synth
    from speculative_verify_attention_amd._binding import _check_accept

    cfg = ACCEPT_WORKLOADS[name]
    n_draft, vocab, temp, with_draft = cfg["n_draft"], cfg["vocab"], cfg["temperature"], cfg["with_draft"]
    torch.cuda.set_device(0)
    rows_t, rows_d = sum(n_draft) + len(n_draft), sum(n_draft)
    # algorithmic bytes: the logits the step must read once (greedy reads
    # only the target rows)
    alg = (rows_t + (rows_d if temp > 0 and with_draft else 0)) * vocab * 4
    reps = max(1, math.ceil((1 << 30) / ((rows_t + rows_d) * vocab * 4)))
    sets = [synth.accept_inputs(n_draft, vocab, 50 + r, "cuda", with_draft=with_draft, boost=4.0) for r in range(reps)]
    need = spec_accept_workspace_bytes(n_draft, vocab, with_draft, temp)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    acc = torch.empty(len(n_draft), dtype=torch.int32, device="cuda")
    tok = torch.empty_like(acc)
    stream = torch.cuda.current_stream()

    def step(i):
        target, draft, tokens, u = sets[i % reps]
        _check_accept(spec_accept(n_draft, target, draft, tokens, u, temp, acc, tok, ws, stream))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stride = event_stride(args.steps)
    ev = {j: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for j in range(0, args.steps, stride)}
    t0 = time.perf_counter()
    for j in range(args.steps):
        if j in ev:
            ev[j][0].record(stream)
        step(args.warmup + j)
        if j in ev:
            ev[j][1].record(stream)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    call_list = [a.elapsed_time(b) for a, b in ev.values()]
    call_ms = sum(call_list) / len(call_list)
    value = rows_d * args.steps / el
    achieved = alg / (call_ms * 1e-3) / 1e9
    res = {
        "metric": "drafts decided/s + logits GB/s (% HBM peak), acceptance step",
        "value": round(value, 2),
        "unit": "drafts decided/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(el * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{name}: {len(n_draft)} seqs x {n_draft[0]} drafts, vocab {vocab}, "
                               f"temperature {temp}, {'draft-model logits' if with_draft else 'point-mass drafts'}",
                   "input_sets": reps, "step": "spec_accept (row statistics, decisions, final draws)"},
        "roofline": {
            "bound": "hbm",
            "kernel": "spec_accept (all three kernels)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "alg_bytes_per_launch": alg,
            "avg_launch_ms": round(call_ms, 5),
            "launch_ms_p10_p50_p90": percentiles(call_list),
            "launches_timed": len(call_list), "event_stride": stride,
        },
    }
    if not args.no_cpu_baseline:
        from oracle import accept as A

        target, draft, tokens, u = [None if x is None else x.cpu() for x in sets[0]]
        tn, dn = target.double().numpy(), None if draft is None else draft.double().numpy()
        kn, un = tokens.numpy(), u.double().numpy()
        calls, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < 10.0:
            A.accept_batch(tn, dn, kn, un, n_draft, temp)
            calls += 1
        cel = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": round(rows_d * calls / cel, 3), "unit": "drafts decided/s",
                               "cores": 1,  # the oracle's per-row softmax and draw are single-threaded numpy
                               "kind": "oracle", "sample": f"the whole call on input set 0, {calls} times in {cel:.1f} s"}
    return res


def describe(name, wl, layers):
    kv = {0: "fp32", 1: "bf16", 2: "tq3 (3-bit Lloyd-Max + QJL keys, 3-bit values)"}[wl.fmt]
    lens = sorted(set(wl.prefill))
    ctx = f"{lens[0]}" if len(lens) == 1 else f"{min(lens)}..{max(lens)} (log-uniform)"
    lay = ", ".join(f"window={w or 'full'}{' (ring cache)' if w else ''} cap={c or 'off'}" for w, c in layers)
    return (f"{name}: {wl.n_seqs} seqs, context {ctx} + drafts, Hq={wl.hq} Hkv={wl.hkv} d={wl.d}, {kv} KV in "
            f"256-token blocks, rows {'1..5 per seq' if wl.vary_rows else wl.rows[0]}, layers [{lay}]")


class Hip:
    """The few HIP runtime calls the timing needs (events)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")

    def event(self):
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(ev))
        assert rc == 0, rc
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        assert rc == 0, rc
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ctypes.c_void_p(ev))


# the sources the attention kernels are built from: counters taken before any
# of them changed no longer describe the kernel
ATTN_SOURCES = ("attn.hip", "attn_tq3.hip", "attn_common.h", "kernels.h")


def source_hash():
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(open(os.path.join(os.path.dirname(ATTN_SRC), f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per launch of the attention kernel from the committed counter
    summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"attn_kernel_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256_16") != source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, layers, budget_s=10.0):
    """The fp64 oracle on this host: whole verify calls for single sequences
    of the workload (all rows and heads), repeated until budget_s passes."""
    import numpy as np
    import torch

    from oracle import attention as A
    from speculative_verify_attention_amd import synth
    from speculative_verify_attention_amd.runner import alg_bytes_per_call

    try:
        from threadpoolctl import threadpool_info

        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas] or [1])
    except Exception:
        threads = 1
    window, cap = max(layers, key=lambda x: x[0] == 0)  # the full-attention layer if any
    s = int(np.argmin(wl.prefill))  # the shortest sequence keeps the sample bounded
    L = wl.prefill[s]
    n = wl.rows[s]
    k, v = synth.prefill_kv(wl, s, 0, L, "cpu")
    k2, v2 = synth.step_kv(wl, 0, n, "cpu")
    k = torch.cat([k, k2]).float().numpy()
    v = torch.cat([v, v2]).float().numpy()
    q = synth.queries(wl, 0, n, "cpu").numpy().astype(np.float64)
    byt_call = alg_bytes_per_call(wl, [n], [L + n], window)
    extra = {}
    if wl.fmt == synth.KV_TQ3:
        # the compressed cache: the oracle encodes the sequence once (untimed;
        # encoding happens on append), then each call decodes every record
        # and runs attention on the decoded values
        from oracle import splitmix, tq3

        signs, s_mat = splitmix.codec_draws(wl.d, wl.codec_seed)
        _, c16, thr = tq3.codebook()
        pi = tq3.rotation(signs)
        ke = tq3.encode_batch(k.reshape(-1, wl.d), True, pi, s_mat, c16, thr)
        ve = tq3.encode_batch(v.reshape(-1, wl.d), False, pi, s_mat, c16, thr)
        shape = (L + n, wl.hkv, wl.d)
        calls, t_dec, t_att, t0 = 0, 0.0, 0.0, time.perf_counter()
        while True:
            ta = time.perf_counter()
            kd = tq3.decode_keys(ke["code"], ke["bits"], ke["n16"], ke["g16"], pi, s_mat, c16).reshape(shape)
            vd = tq3.decode_values(ve["code"], ve["n16"], pi, c16).reshape(shape)
            tb = time.perf_counter()
            A.verify_attention_grouped(q, kd, vd, wl.scale, cap, window)
            t_dec += tb - ta
            t_att += time.perf_counter() - tb
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
        extra = {"decode_s_per_call": round(t_dec / calls, 3), "attention_s_per_call": round(t_att / calls, 3)}
        what = "TQ3 decode of every record + attention"
    else:
        calls, t0 = 0, time.perf_counter()
        while True:
            A.verify_attention_grouped(q, k, v, wl.scale, cap, window)
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
        what = "attention"
    return {
        "value": round(n * calls / el, 3),
        "unit": "verified query-tokens/s",
        "kv_gbs": round(byt_call * calls / el / 1e9, 4),
        "cores": threads,
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"sequence {s} of the workload (context {L}+{n}, {n} rows x {wl.hq} heads): one verify call "
                  f"({what}, fp64) repeated {calls} times in {el:.1f} s",
        **extra,
    }


def run(args, name):
    import torch

    from speculative_verify_attention_amd import kv_workspace_bytes_valu, synth
    from speculative_verify_attention_amd.runner import Runner, alg_bytes_per_call

    wl, layers = workloads()[name]()
    if args.valu:
        args.separate = True  # the vector-unit verify has no fused-append form
    layers = layers or [(wl.window, wl.softcap)]
    total_steps = args.warmup + args.steps
    wl.steps = total_steps  # room in the tables for every step's growth
    torch.cuda.set_device(0)
    dev = "cuda"
    # bytes one layer's cache holds at verify time (stored format)
    per_layer = sum(alg_bytes_per_call(wl, [1], [L + 8], 0) for L in wl.prefill)
    reps = max(1, math.ceil((1 << 30) / max(1, per_layer * len(layers))))
    runners = []
    for _ in range(reps):
        r = Runner(wl, layers=layers, device=dev, ring=True)  # window layers keep their last W + 8 positions
        r.fill()
        runners.append(r)
    # the steps' plans and inputs, generated before timing
    varying = wl.vary_rows or wl.rollback_max
    n_plans = 20 if varying else 1
    plans = [synth.step_plan(wl, t) for t in range(n_plans)]
    inputs = []
    for t, (rb, rows) in enumerate(plans):
        k, v = synth.step_kv(wl, t, sum(rows), dev)
        q = synth.queries(wl, t, sum(rows), dev)
        inputs.append((k, v, q, torch.empty_like(q)))
    seqs = list(range(wl.n_seqs))
    # one workspace per (replica, layer): the partial-slot count is bounded by
    # the workgroup target plus the (sequence, kv head) pairs, whatever the lengths
    ws_need = max(max(runners[0].caches[li].workspace_bytes(seqs, [8] * wl.n_seqs, wl.hq, layers[li][0]),
                      runners[0].caches[li].append_verify_workspace_bytes(seqs, [8] * wl.n_seqs, wl.hq,
                                                                          layers[li][0]),
                      kv_workspace_bytes_valu(runners[0].caches[li].handle, seqs, [8] * wl.n_seqs, wl.hq,
                                              layers[li][0]) if args.valu else 0)
                  for li in range(len(layers)))
    ws = [[torch.empty(2 * ws_need, dtype=torch.uint8, device=dev) for _ in layers] for _ in range(reps)]
    hip = Hip()
    dom = max(range(len(layers)), key=lambda i: layers[i][0] == 0)  # dominant layer: full attention
    stride = event_stride(args.steps)
    ev = {j: (hip.event(), hip.event()) for j in range(0, args.steps, stride)}
    lens = [list(wl.prefill) for _ in range(reps)]  # host-side mirror of seq_len per replica
    last_rows = [None] * reps
    step_bytes = []

    def step(i, timed_idx):
        rep = i % reps
        r = runners[rep]
        t = i % n_plans
        rb, rows = plans[t]
        k, v, q, out = inputs[t]
        if varying:
            back = list(rb)
        else:  # all drafts of this layer's previous step are rejected: the cache returns to its prefill
            back = list(last_rows[rep]) if last_rows[rep] is not None else [0] * wl.n_seqs
        if any(back):
            for c in r.caches:
                c.rollback_batch(seqs, back)
        if args.separate:
            for c in r.caches:
                c.append(seqs, rows, k, v)
        lens[rep] = [L - b + n for L, b, n in zip(lens[rep], back, rows)]
        for li, c in enumerate(r.caches):
            if li == dom and timed_idx in ev:
                c.trace_events(*ev[timed_idx])
            window, cap = layers[li][0], layers[li][1]
            if args.valu:
                c.verify_valu(seqs, rows, q, wl.hq, wl.scale, cap, window, out=out, workspace=ws[rep][li])
            elif args.separate:
                c.verify(seqs, rows, q, wl.hq, wl.scale, cap, window, out=out, workspace=ws[rep][li])
            else:
                c.append_verify(seqs, rows, k, v, q, wl.hq, wl.scale, cap, window, out=out, workspace=ws[rep][li])
            if li == dom and timed_idx in ev:
                c.trace_events(None, None)
        last_rows[rep] = rows
        if timed_idx is not None:
            step_bytes.append([alg_bytes_per_call(wl, rows, lens[rep], w) for w, _ in layers])
        return rows

    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    tok = 0
    t0 = time.perf_counter()
    for j in range(args.steps):
        tok += sum(step(args.warmup + j, j))
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    # sanity: the host mirror of the lengths matches the library's
    for rep in range(reps):
        assert lens[rep] == [runners[rep].caches[0].seq_len(s) for s in seqs]
    kern_ms = [hip.elapsed_ms(a, b) for a, b in ev.values()]
    for a, b in ev.values():
        hip.destroy(a)
        hip.destroy(b)
    kern_avg = sum(kern_ms) / len(kern_ms)
    # bytes of the launches the events timed
    dom_bytes_avg = sum(step_bytes[j][dom] for j in ev) / len(ev)
    byt = sum(sum(b) for b in step_bytes)
    ms_per_step = el * 1e3 / args.steps
    value = tok / el
    kv_gbs = byt / el / 1e9
    achieved = dom_bytes_avg / (kern_avg * 1e-3) / 1e9
    traffic = None if args.valu else load_traffic(name)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "verified query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "f32", 1: "bf16", 2: "f16"}[wl.fmt],
        "data": "synthetic",
        "config": {"workload": describe(name, wl, layers), "layer_replicas": reps,
                   "step": ("rollback previous drafts + append new rows + verify attention (partials + merge)"
                            + (", append and verify as separate calls, products on the vector ALUs "
                               "(spec_verify_attn_valu)" if args.valu else
                               ", append and verify as separate calls" if args.separate else
                               ", append and verify in one call (kv_append_verify)"))},
        "effective_kv_gbs": round(kv_gbs, 2),
        "pct_hbm_peak": round(100.0 * kv_gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": ("attn_valu_kernel" if args.valu else
                       ("attn_tq3_pair_kernel" if wl.d > 128 else "attn_tq3_kernel") if wl.fmt == 2 else "attn_kernel"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": round(dom_bytes_avg),
            "avg_launch_ms": round(kern_avg, 5),
            "launch_ms_p10_p50_p90": percentiles(kern_ms),
            "launches_timed": len(kern_ms), "event_stride": stride,
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, layers)
    return res


def stream_probe(nbytes=2 << 30, runs=10):
    """The library's streaming-read probe (kv_stream_probe) over a buffer far
    larger than the 256 MB Infinity Cache: the read bandwidth a perfect
    single-pass reader of a cache reaches on this GPU.  Returns GB/s (median
    and best of `runs` timed reads, HIP events on the launch stream)."""
    import torch

    from speculative_verify_attention_amd._binding import kv_stream_probe, kv_stream_probe_sink_bytes

    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(kv_stream_probe_sink_bytes() // 4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(2):
        kv_stream_probe(buf, sink, stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    for a, b in ev:
        a.record(stream)
        kv_stream_probe(buf, sink, stream)
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    del buf, sink
    torch.cuda.empty_cache()
    return {"gbs_median": round(nbytes / (ms[len(ms) // 2] * 1e-3) / 1e9, 1),
            "gbs_best": round(nbytes / (ms[0] * 1e-3) / 1e9, 1), "bytes": nbytes, "runs": runs,
            "kernel": "kv_stream_probe (one workgroup per CU, grid-stride 16-byte non-temporal loads, 16 steps in flight)"}


def probe_at_size(nbytes, runs=10, pool=3 << 30):
    """The read probe over `nbytes` (one launch's algorithmic bytes), cycling
    through disjoint slices of a `pool`-byte buffer so that a slice is no
    longer in the 256 MB Infinity Cache when it is read again: how long a
    perfect single-pass reader of that many bytes takes on this GPU, start
    and finish included.  Median of `runs` launches, HIP events."""
    import torch

    from speculative_verify_attention_amd._binding import kv_stream_probe, kv_stream_probe_sink_bytes

    nbytes = int(nbytes) // 16 * 16
    if nbytes <= 0:
        return None
    pool = max(pool, nbytes) // 16 * 16
    buf = torch.ones(pool // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(kv_stream_probe_sink_bytes() // 4, dtype=torch.int32, device="cuda")
    nslice = pool // nbytes
    views = [buf[i * (nbytes // 4):(i + 1) * (nbytes // 4)] for i in range(nslice)]
    stream = torch.cuda.current_stream()
    for v in views[:2]:
        kv_stream_probe(v, sink, stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    for j, (a, b) in enumerate(ev):
        a.record(stream)
        kv_stream_probe(views[j % nslice], sink, stream)
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    del views, buf, sink
    torch.cuda.empty_cache()
    med = ms[len(ms) // 2]
    return {"bytes": nbytes, "us_median": round(med * 1e3, 2), "gbs_median": round(nbytes / (med * 1e-3) / 1e9, 1),
            "slices": nslice, "runs": runs}


def with_probe(res, probe):
    """Fractions of the measured streaming-read bandwidth: of the probe over
    2 GiB, and of the probe over one launch's own byte count (its floor)."""
    ref = probe["gbs_median"]
    r = res["roofline"]
    r["frac_of_stream_probe"] = round(r["achieved"] / ref, 4)
    res["pct_of_stream_probe"] = round(100.0 * res["effective_kv_gbs"] / ref, 2)
    at = probe_at_size(r.get("alg_bytes_per_launch", 0))
    if at:
        r["probe_at_size"] = at
        r["frac_of_probe_at_size"] = round(r["achieved"] / at["gbs_median"], 4)
    return res


def compact(res):
    """The keys of a secondary workload's result carried in the main line."""
    keep = ("value", "unit", "ms_per_step", "dtype", "config", "effective_kv_gbs", "pct_hbm_peak",
            "pct_of_stream_probe", "roofline")
    return {k: res[k] for k in keep if k in res}


def copy_probe(nbytes=1 << 30):
    """A plain elementwise copy of known size (reads nbytes, writes nbytes),
    run before the timed steps so that a counter run can scale the attention
    kernel's HBM byte counters by what they read for a known stream."""
    import torch

    a = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    torch.mul(a, 1, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes}), flush=True)


def _csv_rows(directory, suffix):
    import csv
    import glob

    rows = []
    for f in glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def _layer_pick(workload):
    """(dispatches per step, positions of the dominant layer's) of a
    workload: every step runs the layers in order, each as hs attention
    dispatches (hs head slices: the fewest equal slices of a kv head's query
    group whose columns fit one workgroup, 64 columns, 32 for the compressed
    format at d = 256), so the dominant (full-attention) layer's dispatches
    are positions dom * hs .. dom * hs + hs - 1 of every step."""
    if workload not in workloads():
        return 1, [0]
    wl, layers = workloads()[workload]()
    layers = layers or [(wl.window, wl.softcap)]
    dom = max(range(len(layers)), key=lambda i: layers[i][0] == 0)
    g, cols = wl.hq // wl.hkv, 5 if wl.vary_rows else max(wl.rows)
    cap = 32 if wl.fmt == 2 and wl.d > 128 else 64
    hs = min(h for h in range(1, g + 1) if g % h == 0 and cols * (g // h) <= cap)
    return len(layers) * hs, [dom * hs + j for j in range(hs)]


def _dominant(values, workload, per_call=False):
    """The dominant layer's entries of per-dispatch values in dispatch order:
    every one (per_call=False) or, per call, the sum over its head slices."""
    n, pos = _layer_pick(workload)
    steps = len(values) // n
    if per_call:
        return [sum(values[s * n + p] for p in pos) for s in range(steps)]
    return [values[s * n + p] for s in range(steps) for p in pos]


def _is_attn(name):
    return "attn_kernel" in name or "attn_tq3_kernel" in name or "attn_tq3_pair_kernel" in name or "attn_valu_kernel" in name


def summarize_trace(directory, workload, cmd, out_path=None):
    """profiles/attn_kernel_<workload>_trace.txt from a rocprofv3 --kernel-trace
    --stats run: the library's kernels with calls and durations, and the
    attention dispatches of the dominant (full-attention) layer alone."""
    rows = _csv_rows(directory, "kernel_stats.csv")
    out = [f"# rocprofv3 --kernel-trace --stats summary, workload {workload}",
           f"# command: {cmd}", "# name | calls | average_us | min_us | max_us | percent_of_gpu_time"]
    for r in rows:
        name = r["Name"]
        if "svattn::" not in name:
            continue
        out.append(f"{name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}")
    n_disp, pos = _layer_pick(workload)
    disp = sorted((int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                  for r in _csv_rows(directory, "kernel_trace.csv") if _is_attn(r["Kernel_Name"]))
    if disp:
        d = _dominant([t / 1e3 for _, t in disp], workload, per_call=True)
        out.append(f"# attention dispatches of the dominant layer (positions {pos} of every {n_disp}; one call's "
                   "head slices summed): calls | average_us | min_us | max_us")
        out.append(f"dominant_layer_attention | {len(d)} | {sum(d) / len(d):.2f} | {min(d):.2f} | {max(d):.2f}")
    path = out_path or os.path.join(ROOT, "profiles", f"attn_kernel_{workload}_trace.txt")
    open(path, "w").write("\n".join(out) + "\n")
    return path


def summarize_pmc(fetch_dir, write_dir, workload, cmd_fetch, cmd_write, alg_bytes, out_path=None):
    """profiles/attn_kernel_<workload>_pmc.txt from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for the 1 GiB copy probe."""
    def per_kernel(directory, counter):
        acc = {}
        for r in _csv_rows(directory, "counter_collection.csv"):
            if r.get("Counter_Name") != counter:
                continue
            k = r["Kernel_Name"]
            acc.setdefault(k, []).append((int(r.get("Dispatch_Id", 0)), float(r["Counter_Value"])))
        return acc

    kib = (1 << 30) / 1024.0
    res = {}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        acc = per_kernel(directory, counter)
        attn = _dominant([v for _, v in sorted(x for k, vs in acc.items() if _is_attn(k) for x in vs)], workload,
                         per_call=True)
        acc = {k: [v for _, v in vs] for k, vs in acc.items()}
        copy = [v for k, vs in acc.items() if "MulFunctor" in k or "mul" in k.lower() and "elementwise" in k
                for v in vs if v > kib / 4]
        res[counter] = (sum(attn) / max(1, len(attn)), max(copy) if copy else float("nan"), len(attn))
    f_attn, f_copy, n_f = res["FETCH_SIZE"]
    w_attn, w_copy, n_w = res["WRITE_SIZE"]
    f_scale, w_scale = kib / f_copy, kib / w_copy
    traffic = (f_attn * f_scale + w_attn * w_scale) * 1024.0
    out = [f"# rocprofv3 --pmc summary for the attention kernel, workload {workload}",
           f"# fetch command: {cmd_fetch}", f"# write command: {cmd_write}",
           "# counters are KiB per dispatch, summed over one call's head slices (the dominant, full-attention",
           "# layer's calls only); each is scaled by its reading for a plain copy of 1 GiB",
           f"kernel_sources_sha256_16: {source_hash()}",
           f"attn_dispatches_fetch: {n_f}", f"attn_dispatches_write: {n_w}",
           f"attn_fetch_kib_avg: {f_attn:.1f}", f"copy_fetch_kib: {f_copy:.1f}", f"fetch_scale: {f_scale:.4f}",
           f"attn_write_kib_avg: {w_attn:.1f}", f"copy_write_kib: {w_copy:.1f}", f"write_scale: {w_scale:.4f}",
           f"alg_bytes_per_launch: {alg_bytes}", f"hbm_bytes_per_launch: {traffic:.0f}",
           f"traffic_over_alg: {traffic / alg_bytes:.4f}"]
    path = out_path or os.path.join(ROOT, "profiles", f"attn_kernel_{workload}_pmc.txt")
    open(path, "w").write("\n".join(out) + "\n")
    return path


SQ_PASSES = ("SQ_WAVES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS "
             "SQ_VALU_MFMA_BUSY_CYCLES SQ_WAIT_INST_LDS",
             "SQ_INSTS_MFMA SQ_ACTIVE_INST_VALU SQ_WAIT_INST_ANY SQ_WAVE_CYCLES SQ_INSTS_SALU SQ_INSTS_VMEM_RD "
             "SQ_LDS_ADDR_CONFLICT SQ_ACTIVE_INST_ANY",
             "SQ_INST_LEVEL_LDS SQ_INSTS_LDS SQ_INST_LEVEL_VMEM SQ_INSTS_VMEM_RD SQ_WAIT_ANY SQ_WAVE_CYCLES "
             "SQ_ACTIVE_INST_MISC SQ_ACTIVE_INST_SCA")


def summarize_sq(dirs, workload, cmds, out_path=None):
    """profiles/attn_kernel_<workload>_sq.txt from rocprofv3 --pmc runs of SQ
    counters (instruction mix, waits, matrix-core busy cycles; SQ_PASSES):
    per-dispatch averages of the attention kernel (the dominant layer's
    dispatches) and of the library's other kernels, and per-wave figures of
    the attention kernel."""
    attn, other = {}, {}
    for d in dirs:
        per = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            k = r["Kernel_Name"]
            if "svattn::" not in k:
                continue
            key = (k, r["Counter_Name"])
            per.setdefault(key, {})
            did = int(r["Dispatch_Id"])
            per[key][did] = per[key].get(did, 0.0) + float(r["Counter_Value"])
        counters = sorted({c for _, c in per})
        for c in counters:
            xs = sorted((did, v) for (k, cc), dv in per.items() if cc == c and _is_attn(k) for did, v in dv.items())
            xs = _dominant([v for _, v in xs], workload)
            if xs:
                attn[c] = (sum(xs) / len(xs), len(xs))
            for (k, cc), dv in per.items():
                if cc == c and not _is_attn(k):
                    name = k.split("(")[0].replace("void ", "").replace("svattn::", "")
                    other.setdefault(name, {})[c] = (sum(dv.values()) / len(dv), len(dv))
    out = [f"# rocprofv3 --pmc SQ counter summary, workload {workload}"]
    out += [f"# pass {i + 1} command: {c}" for i, c in enumerate(cmds)]
    out += ["# per-dispatch averages in the units rocprofv3 reports (SQ_ACTIVE_INST_* and SQ_WAVE_CYCLES in",
            "# quad-cycles per wave, summed; SQ_VALU_MFMA_BUSY_CYCLES in cycles summed over the SIMDs);",
            "# attention rows: the dominant (full-attention) layer's dispatches",
            f"kernel_sources_sha256_16: {source_hash()}"]
    if attn:
        out.append(f"== attention kernel ({next(iter(attn.values()))[1]} dispatches)")
        out += [f"  {c:28s} {v:18.1f}" for c, (v, _) in sorted(attn.items())]
        g = {c: v for c, (v, _) in attn.items()}
        waves = g.get("SQ_WAVES", 0.0)
        if waves > 0:
            out.append("== attention kernel, per wave")
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD"):
                if c in g:
                    out.append(f"  {c.lower()[9:] + '_insts_per_wave':28s} {g[c] / waves:18.1f}")
        wc = g.get("SQ_WAVE_CYCLES", 0.0)
        if wc > 0:
            for c in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_MISC",
                      "SQ_ACTIVE_INST_SCA", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_WAIT_INST_LDS"):
                if c in g:
                    out.append(f"  {c.lower()[3:] + '_over_wave_cycles':28s} {g[c] / wc:18.4f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in g:
            out.append(f"  {'mfma_busy_cycles_per_simd':28s} {g['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024:18.1f}")
    for name, cs in sorted(other.items()):
        out.append(f"== {name} ({next(iter(cs.values()))[1]} dispatches)")
        out += [f"  {c:28s} {v:18.1f}" for c, (v, _) in sorted(cs.items())]
    path = out_path or os.path.join(ROOT, "profiles", f"attn_kernel_{workload}_sq.txt")
    open(path, "w").write("\n".join(out) + "\n")
    return path


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=210)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, choices=sorted(workloads()) + sorted(ACCEPT_WORKLOADS),
                    help="one workload; default: tq3_100000 as the line's value, with bf16_100000 beside it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--valu", action="store_true",
                    help="time spec_verify_attn_valu (products on the vector ALUs; bf16 workloads at d 64/128)")
    ap.add_argument("--separate", action="store_true",
                    help="append and verify as two calls (kv_append + spec_verify_attn) instead of kv_append_verify")
    ap.add_argument("--copy-probe", action="store_true", help="run a 1 GiB plain copy first (counter calibration)")
    ap.add_argument("--summarize-trace", metavar="DIR", help="write the profiles/ summary of a kernel-trace run")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summary of two --pmc runs")
    ap.add_argument("--summarize-sq", nargs="+", metavar="DIR",
                    help="write the profiles/ summary of --pmc runs of SQ counters (one directory per pass)")
    ap.add_argument("--cmd", nargs="*", default=[], help="the profiled command(s), recorded in the summary")
    ap.add_argument("--alg-bytes", type=float, default=0.0)
    ap.add_argument("--out", help="summary path (default: profiles/attn_kernel_<workload>_*.txt)")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.workload, " ".join(args.cmd), args.out))
        return
    if args.summarize_sq:
        print(summarize_sq(args.summarize_sq, args.workload, args.cmd, args.out))
        return
    if args.summarize_pmc:
        cmds = args.cmd + ["", ""]
        print(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, cmds[0], cmds[1],
                            args.alg_bytes, args.out))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
    if args.workload in ACCEPT_WORKLOADS:
        print(json.dumps(run_accept(args, args.workload)), flush=True)
        return
    # The long-context compressed and bf16 caches are the headline workloads:
    # the compressed one gives the line's value and roofline, the bf16 one
    # rides along under "also"; --workload NAME times one workload alone.
    main_wl, also = (args.workload, []) if args.workload else ("tq3_100000", ["bf16_100000"])
    res = run(args, main_wl)
    import torch

    torch.cuda.empty_cache()
    extra = {}
    for name in also:
        a = argparse.Namespace(**{**vars(args), "no_cpu_baseline": True})
        extra[name] = run(a, name)
        torch.cuda.empty_cache()
    probe = stream_probe()
    res = with_probe(res, probe)
    if extra:
        res["also"] = {k: compact(with_probe(v, probe)) for k, v in extra.items()}
    res["stream_probe"] = probe
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
