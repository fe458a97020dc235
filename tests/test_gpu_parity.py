"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (written here, per the cache format): fp32 caches 1e-5 max abs
error; bf16 caches 2e-3 max abs error.  Block tables, seq_len and stored
bytes are compared bit for bit.
"""

import math
import os
import zlib

import numpy as np
import pytest
import torch

from parity import max_err, qoffsets, read_plain, require_gpu
from speculative_verify_attention_amd import (KV_BF16, KV_EINVAL, KV_ENOMEM, KV_ENOSEQ, KV_ERANGE, KV_FP32, KVCache,
                                              SvattnError, synth)
from speculative_verify_attention_amd.runner import Runner

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

TOL = {KV_FP32: 1e-5, KV_BF16: 2e-3}


def banner(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def run_and_check(wl, seqs=None, layers=None, scale_q=1.0, steps=(0,), check_steps=None, fused=False, ring=False):
    r = Runner(wl, layers=layers, track=True, ring=ring)
    r.fill()
    worst = 0.0
    for t in steps:
        rows, q, outs = r.step(t, scale_q, fused=fused)
        torch.cuda.synchronize()
        if check_steps is None or t in check_steps:
            for li, out in enumerate(outs):
                e = max_err(r, rows, q, out, li, seqs if seqs is not None else range(wl.n_seqs))
                worst = max(worst, e)
    return r, worst


# ---- the five workloads -----------------------------------------------------------


def test_tiny_fp32():
    banner("tiny fp32 256+5")
    wl = synth.tiny()
    _, err = run_and_check(wl)
    assert err <= TOL[KV_FP32], err


def test_tiny_append5_rollback3_equals_append2():
    banner("tiny append-5/rollback-3 vs append-2")
    wl = synth.tiny()
    a, b = Runner(wl), Runner(wl)
    a.fill()
    b.fill()
    k, v = synth.step_kv(wl, 0, 5, "cuda")
    a.caches[0].append([0], [5], k, v)
    a.caches[0].rollback(0, 3)
    b.caches[0].append([0], [2], k[:2].contiguous(), v[:2].contiguous())
    ca, cb = a.caches[0], b.caches[0]
    assert ca.seq_len(0) == cb.seq_len(0) == 258
    L = ca.seq_len(0)
    assert ca.block_table(0)[: math.ceil(L / 256)] == cb.block_table(0)[: math.ceil(L / 256)]
    ka, va = read_plain(ca, 0, L)
    kb, vb = read_plain(cb, 0, L)
    assert torch.equal(ka.view(torch.int32), kb.view(torch.int32))
    assert torch.equal(va.view(torch.int32), vb.view(torch.int32))
    q = synth.queries(wl, 0, 2, "cuda")
    oa = ca.verify([0], [2], q, wl.hq, wl.scale)
    ob = cb.verify([0], [2], q, wl.hq, wl.scale)
    assert torch.equal(oa, ob)


@pytest.mark.parametrize("fmt", [KV_FP32, KV_BF16])
def test_pool_holds_appended_bits(fmt):
    banner(f"stored bytes fmt={fmt}")
    wl = synth.Workload("bytes", 8, 2, 128, fmt, [300, 513, 7], [3, 1, 5], seed=11, alloc_seed=3)
    r = Runner(wl, track=True)
    r.fill()
    r.step(0)
    torch.cuda.synchronize()
    for s in range(wl.n_seqs):
        L = r.caches[0].seq_len(s)
        assert L == wl.prefill[s] + wl.rows[s]
        k, v = read_plain(r.caches[0], s, L)
        lk, lv = r.logical_kv(s)
        assert np.array_equal(k.float().cpu().numpy(), lk)
        assert np.array_equal(v.float().cpu().numpy(), lv)


def test_qwen3_4b_reduced():
    banner("qwen3-4b dense 3x1000")
    wl = synth.qwen3_4b_dense(batch=3, ctx=1000)
    _, err = run_and_check(wl)
    assert err <= TOL[KV_BF16], err


def test_qwen3_4b_full_separate_calls():
    banner("qwen3-4b dense 16x4096, kv_append + spec_verify_attn, every sequence")
    wl = synth.qwen3_4b_dense()
    _, err = run_and_check(wl)
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL[KV_BF16], err


def test_qwen3_4b_full_fused():
    banner("qwen3-4b dense 16x4096, kv_append_verify (the bench's launch), every sequence")
    wl = synth.qwen3_4b_dense()
    _, err = run_and_check(wl, fused=True)
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL[KV_BF16], err


def test_gemma_interleaved_full_separate_calls():
    banner("gemma 8x32768 window 512 + full, cap 50, separate calls")
    wl = synth.gemma_interleaved()
    _, err = run_and_check(wl, layers=[(512, 50.0), (0, 50.0)])
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL[KV_BF16], err


def test_gemma_interleaved_full_fused_ring():
    banner("gemma 8x32768, window layer on a ring cache + full layer, kv_append_verify (the bench's launch)")
    wl = synth.gemma_interleaved()
    _, err = run_and_check(wl, layers=[(512, 50.0), (0, 50.0)], fused=True, ring=True)
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL[KV_BF16], err


class HostKV:
    """Host copy of a bf16 cache's logical contents, kept step by step
    (rollback = truncate, append = concatenate): the runner's own rebuild
    regenerates every prefill, which is too slow to repeat at every step of
    a 64-sequence batch."""

    def __init__(self, wl):
        self.k, self.v = [], []
        for s, L in enumerate(wl.prefill):
            k, v = synth.prefill_kv(wl, s, 0, L, "cuda")
            self.k.append(k.cpu())
            self.v.append(v.cpu())

    def step(self, rb, rows, k, v):
        k, v = k.cpu(), v.cpu()
        off = 0
        for s, (r, n) in enumerate(zip(rb, rows)):
            L = self.k[s].shape[0] - r
            self.k[s] = torch.cat([self.k[s][:L], k[off: off + n]])
            self.v[s] = torch.cat([self.v[s][:L], v[off: off + n]])
            off += n


@pytest.mark.timeout(1500)
def test_mixed_batch_every_sequence_every_step_fused():
    banner("mixed batch 64 seqs, 20 steps with rollbacks, kv_append_verify, every sequence at every step")
    from oracle import attention as A

    wl = synth.mixed_batch()
    wl.steps = 20
    r = Runner(wl)
    r.fill()
    host = HostKV(wl)
    seqs = list(range(wl.n_seqs))
    worst = 0.0
    for t in range(20):
        rb, rows = synth.step_plan(wl, t)
        r.rollback(rb)
        k, v = synth.step_kv(wl, t, sum(rows), "cuda")
        q = synth.queries(wl, t, sum(rows), "cuda")
        out = r.caches[0].append_verify(seqs, rows, k, v, q, wl.hq, wl.scale)
        torch.cuda.synchronize()
        host.step(rb, rows, k, v)
        qh = q.double().cpu().numpy()
        oh = out.double().cpu().numpy()
        off = qoffsets(rows)
        step_worst = 0.0
        for s in seqs:
            assert r.caches[0].seq_len(s) == host.k[s].shape[0]
            ref = A.verify_attention_grouped(qh[off[s]: off[s + 1]], host.k[s].float().numpy(),
                                             host.v[s].float().numpy(), wl.scale)
            got = oh[off[s]: off[s + 1]]
            assert np.all(np.isfinite(got)), (t, s)
            step_worst = max(step_worst, float(np.max(np.abs(got - ref))))
        worst = max(worst, step_worst)
        print(f"step {t}: rows {sum(rows)}, max abs err {step_worst:.3e}", flush=True)
    assert worst <= TOL[KV_BF16], worst


@pytest.mark.timeout(900)
def test_bf16_long_context_every_sequence_fused():
    banner("bf16 4x100000, kv_append_verify (the bench's launch), every sequence")
    wl = synth.tq3_long(100000, fmt=KV_BF16)
    _, err = run_and_check(wl, fused=True)
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL[KV_BF16], err


def test_library_loaded_from_tree():
    banner("the library mapped into this process is the in-tree build")
    from speculative_verify_attention_amd import _binding

    wl = synth.tiny()
    Runner(wl).fill()
    maps = open("/proc/self/maps").read()
    assert _binding.LIB_PATH in maps
    assert os.path.dirname(_binding.LIB_PATH) == os.path.join(ROOT, "speculative_verify_attention_amd")


@pytest.mark.parametrize("nbytes", [16, 4096 * 256 * 16 + 48, 4 << 20])
def test_stream_probe_reads_every_word(nbytes):
    # the probe folds every 32-bit word of the buffer into the sink exactly
    # once (xor), so the xor of the sink words is the xor of the buffer
    banner(f"kv_stream_probe over {nbytes} bytes")
    import numpy as np

    from speculative_verify_attention_amd import _binding

    g = torch.Generator(device="cpu")
    g.manual_seed(nbytes)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4,), generator=g, dtype=torch.int64).to(torch.int32)
    src = host.cuda()
    sink = torch.full((_binding.kv_stream_probe_sink_bytes() // 4,), -1, dtype=torch.int32, device="cuda")
    _binding.kv_stream_probe(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert int(got) == int(want)


def test_stream_probe_rejects_bad_arguments():
    banner("kv_stream_probe argument checks")
    from speculative_verify_attention_amd import _binding

    src = torch.zeros(64, dtype=torch.int32, device="cuda")
    sink = torch.zeros(_binding.kv_stream_probe_sink_bytes() // 4, dtype=torch.int32, device="cuda")
    with pytest.raises(SvattnError) as ei:
        _binding.kv_stream_probe(src[:3], sink)  # 12 bytes: not a multiple of 16
    assert ei.value.code == KV_EINVAL
    with pytest.raises(SvattnError) as ei:
        _binding.kv_stream_probe(src, sink[:4])  # sink too small
    assert ei.value.code == KV_EINVAL


# ---- edge cases -----------------------------------------------------------------------


EDGE = [
    # name, hq, hkv, d, fmt, prefill, rows, window, cap, scale_q
    ("plain_decode", 8, 2, 128, KV_BF16, [700, 64, 1], [1, 1, 1], 0, 0.0, 1.0),
    ("max_rows", 8, 2, 64, KV_FP32, [300, 40], [8, 8], 0, 0.0, 1.0),
    ("context_equals_rows", 4, 1, 64, KV_FP32, [0, 0], [5, 1], 0, 0.0, 1.0),
    ("mha_g1", 4, 4, 128, KV_BF16, [333], [5], 0, 0.0, 1.0),
    ("two_column_groups", 24, 2, 128, KV_BF16, [1000, 77], [5, 5], 0, 0.0, 1.0),
    ("two_column_groups_fp32", 24, 2, 64, KV_FP32, [200, 5], [5, 2], 0, 0.0, 1.0),
    ("window_1", 8, 2, 64, KV_FP32, [500], [5], 1, 0.0, 1.0),
    ("window_ge_ctx", 8, 2, 128, KV_BF16, [400], [5], 100000, 0.0, 1.0),
    ("window_ragged", 8, 1, 256, KV_BF16, [3000, 70], [5, 3], 100, 0.0, 1.0),
    ("softcap_saturating", 8, 1, 256, KV_BF16, [900], [5], 0, 50.0, 20.0),
    ("softcap_fp32", 8, 2, 64, KV_FP32, [600], [4], 0, 5.0, 3.0),
    ("d256_fp32", 8, 2, 256, KV_FP32, [300], [5], 0, 0.0, 1.0),
    ("d64_bf16", 16, 4, 64, KV_BF16, [5000, 1], [5, 1], 0, 0.0, 1.0),
    ("many_seqs", 8, 2, 128, KV_BF16, [int(x) for x in np.linspace(1, 3000, 150)], [2] * 150, 0, 0.0, 1.0),
    # one (sequence, kv head) pair split into more than 64 chunks: the merge
    # folds chunks past the wave's 64 lanes
    ("single_pair_long", 8, 1, 128, KV_BF16, [60000], [5], 0, 0.0, 1.0),
    # sharp scores from fp32 queries that bf16 cannot represent (the kernel
    # carries the query as two bf16 parts)
    ("sharp_fp32_queries", 32, 8, 128, KV_BF16, [3000, 500], [5, 5], 0, 0.0, 4.0),
    ("sharp_fp32_queries_d256", 8, 1, 256, KV_BF16, [2000], [5], 0, 0.0, 3.0),
    ("sharp_fp32_queries_d64", 16, 4, 64, KV_BF16, [1500], [4], 0, 0.0, 5.0),
    # more than 64 query columns per kv head: the call splits the group's
    # heads into slices (5 x 16 = 80 -> 2 x 8 heads; 8 x 12 = 96 -> 2 x 6;
    # 8 x 64 = 512 -> 8 x 8, with a window, a cap and sharp scores)
    ("head_slices_g16", 32, 2, 128, KV_BF16, [900, 300], [5, 4], 0, 0.0, 1.0),
    ("head_slices_g12_fp32", 12, 1, 64, KV_FP32, [400, 9], [8, 8], 0, 0.0, 1.0),
    ("head_slices_g64_window_cap", 64, 1, 128, KV_BF16, [700, 20], [8, 3], 100, 30.0, 2.0),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge(case):
    name, hq, hkv, d, fmt, prefill, rows, window, cap, scale_q = case
    banner(f"edge {name}")
    wl = synth.Workload(name, hq, hkv, d, fmt, prefill, rows, window=window, softcap=cap, seed=zlib.crc32(name.encode()) % 1000,
                        alloc_seed=17)
    _, err = run_and_check(wl, scale_q=scale_q)
    assert err <= TOL[fmt], err


def test_window_1_returns_own_value_exactly():
    banner("window 1 exact")
    wl = synth.Workload("w1", 8, 2, 64, KV_FP32, [260], [5], window=1, seed=5)
    r = Runner(wl, track=True)
    r.fill()
    rows, q, (out,) = r.step(0)
    k, v = r.logical_kv(0)
    o = out.cpu().numpy()
    for i in range(5):
        for h in range(8):
            assert np.array_equal(o[i, h], v[260 + i, h // 4])


def test_deterministic():
    banner("determinism")
    wl = synth.qwen3_4b_dense(batch=4, ctx=2000)
    r = Runner(wl)
    r.fill()
    rows, q, (o1,) = r.step(0)
    o2 = r.verify(0, rows, q)
    o3 = r.verify(0, rows, q)
    assert torch.equal(o1, o2) and torch.equal(o2, o3)


def test_errors_change_nothing():
    banner("error returns")
    wl = synth.Workload("err", 8, 2, 64, KV_BF16, [100, 3], [5, 5], seed=1)
    r = Runner(wl)
    r.fill()
    c = r.caches[0]
    q = synth.queries(wl, 0, 16, "cuda")
    out = torch.zeros_like(q)
    before = (c.seq_len(0), c.seq_len(1), c.block_table(0), c.free_blocks())

    def code_of(fn):
        with pytest.raises(SvattnError) as e:
            fn()
        return e.value.code

    assert code_of(lambda: c.verify([0, 1], [5, 11], q, 8, 0.1, out=out)) == KV_EINVAL  # > KV_MAX_ROWS rows
    assert code_of(lambda: c.verify([0, 1], [5, 5], q, 8, 0.1, out=out)) == KV_ERANGE  # 5 rows, 3 positions
    assert code_of(lambda: c.verify([0, 9], [5, 2], q, 8, 0.1, out=out)) == KV_ENOSEQ
    q7 = torch.zeros((16, 7, 64), device="cuda")
    assert code_of(lambda: c.verify([0], [5], q7, 7, 0.1, out=torch.zeros_like(q7))) == KV_EINVAL  # 7 % 2 != 0
    small_ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    assert code_of(lambda: c.verify([0], [5], q, 8, 0.1, out=out, workspace=small_ws)) == KV_ENOMEM
    assert code_of(lambda: c.verify([0], [5], q, 8, float("nan"), out=out)) == KV_EINVAL
    assert code_of(lambda: c.verify([0], [5], q, 8, 0.1, softcap=-1.0, out=out)) == KV_EINVAL
    assert code_of(lambda: c.verify([0], [5], q, 8, 0.1, window=-3, out=out)) == KV_EINVAL
    assert code_of(lambda: c.rollback(1, 4)) == KV_ERANGE
    assert code_of(lambda: c.rollback(1, -1)) == KV_EINVAL
    assert code_of(lambda: c.rollback(5, 1)) == KV_ENOSEQ
    big = torch.zeros((10000, 2, 64), dtype=torch.bfloat16, device="cuda")
    assert code_of(lambda: c.append([1], [10000], big, big)) in (KV_ENOMEM, KV_ERANGE)
    assert code_of(lambda: c.append([0, 0], [1, 1], big, big)) == KV_EINVAL
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
    assert (c.seq_len(0), c.seq_len(1), c.block_table(0), c.free_blocks()) == before
