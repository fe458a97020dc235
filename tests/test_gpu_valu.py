"""GPU parity of the vector-unit verify (spec_verify_attn_valu) through the C
ABI: the same call as spec_verify_attn with its products on the vector ALUs
(the measurement twin of the matrix-core kernel for the MFMA-or-VALU
choice).  Bars: the fp64 oracle at 2e-3 (bf16 caches), as for the
matrix-core path, and agreement with the matrix-core path's output on the
same cache to 1e-4 (both carry the queries and probabilities as two bf16
parts, so only the summation order differs)."""

import zlib

import numpy as np
import pytest
import torch

from parity import max_err, require_gpu
from speculative_verify_attention_amd import KV_BF16, KV_EINVAL, KV_FP32, KV_TQ3, SvattnError, synth
from speculative_verify_attention_amd.runner import Runner

pytestmark = pytest.mark.gpu

TOL = 2e-3
TWIN = 1e-4


def banner(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def check(wl, layers=None, scale_q=1.0, seqs=None, steps=(0,)):
    r = Runner(wl, layers=layers, track=True)
    r.fill()
    worst, gap = 0.0, 0.0
    for t in steps:
        rows, q, outs = r.step(t, scale_q)
        for li, (window, cap) in enumerate(r.layers):
            c = r.caches[li]
            ov = c.verify_valu(list(range(wl.n_seqs)), rows, q, wl.hq, wl.scale, cap, window)
            torch.cuda.synchronize()
            gap = max(gap, float((ov - outs[li]).abs().max()))
            worst = max(worst, max_err(r, rows, q, ov, li, seqs if seqs is not None else range(wl.n_seqs)))
    print(f"max abs err vs oracle {worst:.3e}, vs the matrix-core path {gap:.3e}", flush=True)
    assert worst <= TOL, worst
    assert gap <= TWIN, gap


# name, hq, hkv, d, prefill, rows, layers [(window, cap)], scale_q
CASES = [
    ("gqa_d128", 32, 8, 128, [1000, 77, 3], [5, 3, 1], None, 1.0),
    ("d64", 16, 4, 64, [900, 5], [5, 2], None, 1.0),
    ("odd_subtile_count", 8, 2, 128, [32 * 7 + 5, 64 * 3], [4, 5], None, 1.0),
    ("window_and_cap", 8, 1, 128, [2000, 300], [5, 4], [(100, 30.0), (0, 30.0)], 2.0),
    ("sharp_scores", 32, 8, 128, [3000], [5], None, 4.0),
    ("mha", 4, 4, 128, [500], [8], None, 1.0),
    # 5 rows x a group of 16 = 80 columns: head slices of 4 heads (20 columns)
    ("head_slices_g16", 32, 2, 128, [700, 90], [5, 4], None, 1.0),
    ("many_seqs", 8, 2, 64, [int(x) for x in np.linspace(1, 1500, 140)], [2] * 140, None, 1.0),
    ("single_pair_long", 8, 1, 128, [40000], [5], None, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_valu_matches_oracle(case):
    name, hq, hkv, d, prefill, rows, layers, scale_q = case
    banner(f"valu {name}")
    wl = synth.Workload(name, hq, hkv, d, KV_BF16, prefill, rows, seed=zlib.crc32(name.encode()) % 1000, alloc_seed=5)
    check(wl, layers=layers, scale_q=scale_q)


def test_valu_qwen3_4b_full():
    banner("valu qwen3-4b dense 16x4096, every sequence")
    check(synth.qwen3_4b_dense())


@pytest.mark.timeout(900)
def test_valu_bf16_100000_full():
    banner("valu bf16 4x100000, every sequence")
    check(synth.tq3_long(100000, fmt=KV_BF16))


def test_valu_rejects_other_formats():
    banner("valu refuses fp32, TQ3 and head_dim 256")
    for fmt, d in ((KV_FP32, 128), (KV_TQ3, 128), (KV_BF16, 256)):
        wl = synth.Workload("rej", 8, 2, d, fmt, [100], [5], seed=1, codec_seed=0x5EED)
        r = Runner(wl)
        r.fill()
        rows, q, _ = r.step(0)
        with pytest.raises(SvattnError) as ei:
            r.caches[0].verify_valu([0], rows, q, wl.hq, wl.scale)
        assert ei.value.code == KV_EINVAL
