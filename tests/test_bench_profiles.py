"""bench.py's rocprofv3 summaries on synthetic CSV files (no GPU): the
counter summary scales FETCH_SIZE and WRITE_SIZE by their readings for the
1 GiB copy probe; the trace and SQ summaries keep only the dominant
(full-attention) layer's attention dispatches, which alternate with the
window layer's in the two-layer workload."""

import csv
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

ATTN = "void svattn::attn_kernel<1, 256, 2, true, true>(svattn::AttnArgs)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<int>>(int, at::native::MulFunctor<int>)"
MERGE = "void svattn::merge_kernel<256, false>(svattn::AttnArgs)"


def write_csv(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def counters(path, per_dispatch):
    """per_dispatch: [(dispatch id, kernel, counter, value)]"""
    write_csv(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
              [dict(Dispatch_Id=d, Kernel_Name=k, Counter_Name=c, Counter_Value=v) for d, k, c, v in per_dispatch])


def fields_of(path):
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    return vals


def test_pmc_summary_scales_by_the_copy_probe(tmp_path):
    # one-layer workload: every attention dispatch counts; the copy reads
    # 0.5 GiB of FETCH_SIZE and 1 GiB of WRITE_SIZE for a 1 GiB copy
    f_dir, w_dir = tmp_path / "f", tmp_path / "w"
    counters(str(f_dir / "pmc_counter_collection.csv"),
             [(1, COPY, "FETCH_SIZE", 524288.0)] + [(2 + i, ATTN, "FETCH_SIZE", 1000.0 + 10 * i) for i in range(5)])
    counters(str(w_dir / "pmc_counter_collection.csv"),
             [(1, COPY, "WRITE_SIZE", 1048576.0)] + [(2 + i, ATTN, "WRITE_SIZE", 50.0) for i in range(5)])
    out = str(tmp_path / "pmc.txt")
    bench.summarize_pmc(str(f_dir), str(w_dir), "qwen3_4b_dense", "c1", "c2", 1_000_000, out)
    v = fields_of(out)
    assert float(v["fetch_scale"]) == 2.0 and float(v["write_scale"]) == 1.0
    want = (1020.0 * 2.0 + 50.0) * 1024.0  # mean fetch of 1000..1040 KiB
    assert abs(float(v["hbm_bytes_per_launch"]) - want) < 1.0
    assert abs(float(v["traffic_over_alg"]) - want / 1e6) < 1e-4
    assert v["kernel_sources_sha256_16"] == bench.source_hash()


def test_trace_summary_keeps_the_dominant_layer(tmp_path):
    # two-layer workload: window layer first, then the full layer, per step
    d = tmp_path / "t"
    write_csv(str(d / "kt_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
              [dict(Name=ATTN, Calls=8, AverageNs=40000, MinNs=9000, MaxNs=72000, Percentage=90.0),
               dict(Name=MERGE, Calls=8, AverageNs=4000, MinNs=3500, MaxNs=4500, Percentage=10.0)])
    rows = []
    for i in range(8):
        dur = 10_000 if i % 2 == 0 else 70_000 + 1000 * i  # ns: window, full
        rows.append(dict(Dispatch_Id=10 + 2 * i, Kernel_Name=ATTN, Start_Timestamp=1_000_000 * i,
                         End_Timestamp=1_000_000 * i + dur))
        rows.append(dict(Dispatch_Id=11 + 2 * i, Kernel_Name=MERGE, Start_Timestamp=1_000_000 * i + 500_000,
                         End_Timestamp=1_000_000 * i + 504_000))
    write_csv(str(d / "kt_kernel_trace.csv"), ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    out = str(tmp_path / "trace.txt")
    bench.summarize_trace(str(d), "gemma_interleaved", "cmd", out)
    line = [x for x in open(out) if x.startswith("dominant_layer_attention")][0]
    _, calls, avg, lo, hi = [x.strip() for x in line.split("|")]
    assert int(calls) == 4
    assert float(avg) == 74.0 and float(lo) == 71.0 and float(hi) == 77.0  # 71, 73, 75, 77 us


def test_trace_summary_sums_head_slices(tmp_path):
    # compressed cache at d = 256 with 5 rows x 8 heads = 40 columns: two head
    # slices per call, so a step is window slice 0, 1, then full slice 0, 1
    tq3 = "void svattn::attn_tq3_kernel<256, 1, true>(svattn::AttnArgs)"
    d = tmp_path / "t"
    write_csv(str(d / "kt_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
              [dict(Name=tq3, Calls=12, AverageNs=30000, MinNs=5000, MaxNs=60000, Percentage=100.0)])
    rows = []
    for s in range(3):
        for j, dur in enumerate((5_000, 6_000, 50_000 + 1000 * s, 52_000 + 1000 * s)):
            i = 4 * s + j
            rows.append(dict(Dispatch_Id=10 + i, Kernel_Name=tq3, Start_Timestamp=1_000_000 * i,
                             End_Timestamp=1_000_000 * i + dur))
    write_csv(str(d / "kt_kernel_trace.csv"), ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    out = str(tmp_path / "trace.txt")
    assert bench._layer_pick("gemma_tq3") == (4, [2, 3])
    bench.summarize_trace(str(d), "gemma_tq3", "cmd", out)
    line = [x for x in open(out) if x.startswith("dominant_layer_attention")][0]
    _, calls, avg, lo, hi = [x.strip() for x in line.split("|")]
    assert int(calls) == 3
    assert float(lo) == 102.0 and float(avg) == 104.0 and float(hi) == 106.0  # 50+52, 51+53, 52+54 us


def test_sq_summary_per_wave_figures(tmp_path):
    a, b = tmp_path / "a", tmp_path / "b"
    p1, p2 = [], []
    for i in range(6):
        full = i % 2 == 1  # dispatches alternate window, full
        p1 += [(20 + 2 * i, ATTN, "SQ_WAVES", 1024.0),
               (20 + 2 * i, ATTN, "SQ_INSTS_VALU", 1024.0 * (3000.0 if full else 100.0)),
               (21 + 2 * i, MERGE, "SQ_WAVES", 640.0)]
        p2 += [(20 + 2 * i, ATTN, "SQ_WAVE_CYCLES", 4000.0 if full else 50.0),
               (20 + 2 * i, ATTN, "SQ_ACTIVE_INST_VALU", 1000.0 if full else 40.0)]
    counters(str(a / "pmc_counter_collection.csv"), p1)
    counters(str(b / "pmc_counter_collection.csv"), p2)
    out = str(tmp_path / "sq.txt")
    bench.summarize_sq([str(a), str(b)], "gemma_interleaved", ["c1", "c2"], out)
    text = open(out).read()
    per = {}
    for line in text.splitlines():
        parts = line.split()
        if len(parts) == 2 and line.startswith("  ") and parts[0].islower():
            per[parts[0]] = float(parts[1])
    assert per["valu_insts_per_wave"] == 3000.0
    assert per["active_inst_valu_over_wave_cycles"] == 0.25
    assert "== attention kernel (3 dispatches)" in text
    assert "== merge_kernel<256, false> (6 dispatches)" in text


def test_every_attention_kernel_is_counted():
    """The summaries count the dispatches of every partial-attention kernel
    the library launches (plain, TQ3 one-wave, TQ3 wave-pair, vector-unit)
    and of nothing else."""
    for name in ("void svattn::attn_kernel<1, 128, 1, false, true>(svattn::AttnArgs)",
                 "void svattn::attn_tq3_kernel<128, 1, false>(svattn::AttnArgs)",
                 "void svattn::attn_tq3_pair_kernel<true>(svattn::AttnArgs)",
                 "void svattn::attn_valu_kernel<128, false>(svattn::AttnArgs)"):
        assert bench._is_attn(name), name
    for name in ("void svattn::merge_kernel<256, true>(svattn::AttnArgs)",
                 "void svattn::append_tq3_kernel<256>(svattn::AppendArgs)",
                 "void svattn::append_tq3_qprep_kernel<256>(svattn::AppendArgs, svattn::QPrepArgs, int)",
                 "void svattn::stream_probe_kernel<16>(unsigned int __vector(4) const*, long, unsigned int*)"):
        assert not bench._is_attn(name), name
