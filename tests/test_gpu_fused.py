"""GPU tests of the fused append + verify call (kv_append_verify) and of
device-side rollback (kv_rollback_device / kv_sync), through the C ABI.

Both reorganise work the separate calls already do, so each run drives two
caches with the same inputs: a twin with kv_append + spec_verify_attn and
host rollbacks, and the cache under test.  Bars:
* fused call, host rollbacks: outputs, lengths, block tables and stored bytes
  bit-identical to the twin's;
* device rollbacks: lengths and stored bytes of the live positions
  bit-identical after kv_sync; outputs within 2e-5 of the twin's at every
  step (the host plans the split from upper bounds of the lengths, so the
  partials are summed in another order);
* and, for the cache under test, the final step's outputs against the fp64
  oracle (1e-5 for fp32 and TQ3 caches, 2e-3 for bf16), on the logical
  contents its own appends and rollbacks define.
"""

import math

import numpy as np
import pytest
import torch

from parity import max_err, max_err_tq3, read_plain, read_tq3, require_gpu
from speculative_verify_attention_amd import (KV_BF16, KV_EINVAL, KV_ERANGE, KV_FP32, KV_TQ3, SvattnError, synth)
from speculative_verify_attention_amd.runner import Runner

pytestmark = pytest.mark.gpu

TOL = {KV_FP32: 1e-5, KV_BF16: 2e-3, KV_TQ3: 1e-5}
STEPS = 12


def banner(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def workload(fmt, hq, hkv, d, prefill, window=0, cap=0.0, seed=11, alloc_seed=0xB10C5):
    return synth.Workload("fused", hq, hkv, d, fmt, list(prefill), [5] * len(prefill), window=window, softcap=cap,
                          seed=seed, alloc_seed=alloc_seed, codec_seed=0x5EED, steps=STEPS + 2)


def plan(wl, t):
    """Rows (1 + drafts) per sequence and accepted drafts, seeded per step."""
    rng = np.random.default_rng(1000 + 17 * wl.seed + t)
    rows = rng.integers(1, 6, size=wl.n_seqs)
    acc = np.array([rng.integers(0, r) for r in rows])  # 0 .. drafts
    return rows.tolist(), acc.tolist()


def track_append(r, k, v, rows):
    r.step_k.append(k.float().cpu().numpy())
    r.step_v.append(v.float().cpu().numpy())
    off = r.step_rows0
    for s, n in enumerate(rows):
        r.prov[s] = np.concatenate([r.prov[s], off + np.arange(n, dtype=np.int64)])
        off += n
    r.step_rows0 = off


def track_rollback(r, rb):
    for s, b in enumerate(rb):
        if b:
            r.prov[s] = r.prov[s][: len(r.prov[s]) - b]


def oracle_err(r, rows, q, out, li):
    f = max_err_tq3 if r.wl.fmt == KV_TQ3 else max_err
    return f(r, rows, q, out, li, range(r.wl.n_seqs))


def stored(cache, s, L):
    if cache.fmt == KV_TQ3:
        return read_tq3(cache, s, L)
    k, v = read_plain(cache, s, L)
    return {"k": k.view(torch.int16 if cache.fmt == KV_BF16 else torch.int32).cpu().numpy(),
            "v": v.view(torch.int16 if cache.fmt == KV_BF16 else torch.int32).cpu().numpy()}


def run_twins(wl, layers, fused, device_rb, steps=STEPS):
    """Drive the twin (separate calls, host rollbacks) and the cache under
    test; returns (twin, test, worst output gap per step, last rows/q/outs)."""
    seqs = list(range(wl.n_seqs))
    a = Runner(wl, layers=layers, track=True)
    b = Runner(wl, layers=layers, track=True)
    a.fill()
    b.fill()
    gaps = []
    last = None
    for t in range(steps):
        rows, acc = plan(wl, t)
        drafts = [n - 1 for n in rows]
        rb = [d - x for d, x in zip(drafts, acc)]
        k, v = a.append_rows(t, rows)
        q = a.queries(t, rows)
        outs_a = [a.verify(li, rows, q) for li in range(len(layers))]
        outs_b = []
        for li, c in enumerate(b.caches):
            window, cap = layers[li]
            if fused:
                outs_b.append(c.append_verify(seqs, rows, k, v, q, wl.hq, wl.scale, cap, window))
            else:
                c.append(seqs, rows, k, v)
                outs_b.append(c.verify(seqs, rows, q, wl.hq, wl.scale, cap, window))
        track_append(b, k, v, rows)
        torch.cuda.synchronize()
        gaps.append(max(float((x - y).abs().max()) for x, y in zip(outs_a, outs_b)))
        last = (rows, q, outs_b)
        if t == steps - 1:
            break  # the final outputs are checked against the oracle before any rollback
        a.rollback(rb)
        if device_rb:
            acc_dev = torch.tensor(acc, dtype=torch.int32, device="cuda")
            for c in b.caches:
                c.rollback_device(seqs, drafts, acc_dev)
            track_rollback(b, rb)
        else:
            b.rollback(rb)
    return a, b, gaps, last


def check_run(wl, layers, fused, device_rb):
    a, b, gaps, (rows, q, outs) = run_twins(wl, layers, fused, device_rb)
    worst = max(gaps)
    print(f"max |test - twin| over {len(gaps)} steps: {worst:.3e}", flush=True)
    if device_rb:
        assert worst <= 2e-5, gaps
    else:
        assert worst == 0.0, gaps
    for li in range(len(layers)):
        err = oracle_err(b, rows, q, outs[li], li)
        print(f"layer {li}: max abs err vs oracle {err:.3e}", flush=True)
        assert err <= TOL[wl.fmt], err
    for ca, cb in zip(a.caches, b.caches):
        cb.sync()
        for s in range(wl.n_seqs):
            L = ca.seq_len(s)
            assert cb.seq_len(s) == L == len(b.prov[s])
            if not device_rb:  # host reservations see the same lengths: the same blocks
                assert ca.block_table(s)[: math.ceil(L / 256)] == cb.block_table(s)[: math.ceil(L / 256)]
            xa, xb = stored(ca, s, L), stored(cb, s, L)
            for key in xa:
                assert np.array_equal(np.asarray(xa[key]), np.asarray(xb[key])), (s, key)


# name, fmt, hq, hkv, d, prefill, layers [(window, cap)]
CASES = [
    ("fp32_d64", KV_FP32, 8, 2, 64, [250, 509, 3, 1000, 767], [(0, 0.0)]),
    ("bf16_gqa_d128", KV_BF16, 32, 8, 128, [251, 40, 1023, 600], [(0, 0.0)]),
    ("bf16_d256_window_cap", KV_BF16, 8, 1, 256, [300, 700, 62], [(64, 50.0), (0, 50.0)]),
    ("bf16_d64_two_groups", KV_BF16, 24, 2, 64, [255, 90], [(0, 0.0)]),
    ("tq3_d128", KV_TQ3, 8, 2, 128, [250, 509, 33], [(0, 0.0)]),
    ("tq3_d64_window", KV_TQ3, 8, 1, 64, [700, 40], [(64, 0.0)]),
    # a group of 16: steps with 5 rows split the heads into two slices
    ("bf16_g16_head_slices", KV_BF16, 32, 2, 128, [250, 700, 31], [(0, 0.0)]),
    ("tq3_g16_head_slices", KV_TQ3, 32, 2, 128, [300, 90], [(0, 0.0)]),
    ("tq3_d256_window_cap", KV_TQ3, 8, 1, 256, [300, 700, 62], [(64, 50.0), (0, 0.0)]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_append_verify_equals_separate_calls(case):
    name, fmt, hq, hkv, d, prefill, layers = case
    banner(f"append_verify {name}")
    check_run(workload(fmt, hq, hkv, d, prefill), layers, fused=True, device_rb=False)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_device_rollback(case):
    name, fmt, hq, hkv, d, prefill, layers = case
    banner(f"device rollback + append_verify {name}")
    check_run(workload(fmt, hq, hkv, d, prefill, seed=23), layers, fused=True, device_rb=True)


def test_device_rollback_with_separate_calls():
    banner("device rollback + kv_append / spec_verify_attn")
    wl = workload(KV_BF16, 16, 4, 128, [250, 511, 20, 900])
    check_run(wl, [(0, 0.0)], fused=False, device_rb=True)


def test_many_sequences_fused():
    banner("append_verify, 150 sequences (two launches)")
    wl = workload(KV_BF16, 8, 2, 64, [int(x) for x in np.linspace(5, 1200, 150)], seed=31)
    a, b, gaps, _ = run_twins(wl, [(0, 0.0)], fused=True, device_rb=False, steps=3)
    assert max(gaps) == 0.0


def test_seq_len_applies_pending_rollbacks():
    banner("kv_seq_len after kv_rollback_device")
    wl = workload(KV_BF16, 8, 2, 64, [100, 300])
    r = Runner(wl)
    r.fill()
    c = r.caches[0]
    k, v = synth.step_kv(wl, 0, 8, "cuda")
    q = synth.queries(wl, 0, 8, "cuda")
    c.append_verify([0, 1], [5, 3], k, q=q, v=v, num_q_heads=wl.hq, scale=wl.scale)
    c.rollback_device([0, 1], [4, 2], torch.tensor([1, 2], dtype=torch.int32, device="cuda"))
    assert c.seq_len(0) == 100 + 5 - 3
    assert c.seq_len(1) == 300 + 3 - 0
    c.sync()  # nothing pending: a no-op
    assert c.seq_len(0) == 102


def test_device_rollback_errors_change_nothing():
    banner("kv_rollback_device argument errors")
    wl = workload(KV_BF16, 8, 2, 64, [10, 20])
    r = Runner(wl)
    r.fill()
    c = r.caches[0]
    acc = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(SvattnError) as e:
        c.rollback_device([0, 1], [11, 1], acc)  # more drafts than positions
    assert e.value.code == KV_ERANGE
    with pytest.raises(SvattnError) as e:
        c.rollback_device([1, 1], [1, 1], acc)
    assert e.value.code == KV_EINVAL
    c.rollback_device([0], [4], acc)  # rolls back 4 on the current stream
    other = torch.cuda.Stream()
    with pytest.raises(SvattnError) as e:
        c.rollback_device([1], [1], acc, stream=other)  # pending work sits on another stream
    assert e.value.code == KV_EINVAL
    # a pending rollback bounds what a verify may ask for: 10 - 4 = 6 positions left
    q = synth.queries(wl, 0, 8, "cuda")
    with pytest.raises(SvattnError) as e:
        c.verify([0], [8], q, wl.hq, wl.scale)
    assert e.value.code == KV_ERANGE
    assert c.seq_len(0) == 6 and c.seq_len(1) == 20


def test_append_verify_errors_change_nothing():
    banner("append_verify argument errors")
    from speculative_verify_attention_amd import KV_ENOMEM

    wl = workload(KV_BF16, 8, 2, 64, [250, 40])
    r = Runner(wl)
    r.fill()
    c = r.caches[0]
    snap = lambda: ([c.seq_len(s) for s in (0, 1)], [c.block_table(s) for s in (0, 1)], c.free_blocks())  # noqa: E731
    before = snap()
    k, v = synth.step_kv(wl, 0, 8, "cuda")
    q = synth.queries(wl, 0, 8, "cuda")
    with pytest.raises(SvattnError) as e:
        c.append_verify([0, 1], [5, 0], k, v, q, wl.hq, wl.scale)  # a verify needs >= 1 row
    assert e.value.code == KV_EINVAL
    k16, v16 = synth.step_kv(wl, 1, 16, "cuda")
    q16 = synth.queries(wl, 1, 16, "cuda")
    with pytest.raises(SvattnError) as e:
        c.append_verify([0, 1], [5, 9], k16, v16, q16, wl.hq, wl.scale)  # more rows than a call verifies
    assert e.value.code == KV_EINVAL
    tiny = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(SvattnError) as e:
        c.append_verify([0, 1], [5, 3], k, v, q, wl.hq, wl.scale, workspace=tiny)
    assert e.value.code == KV_ENOMEM
    assert snap() == before  # no append was committed by any failed call


def test_append_verify_unaligned_rows_take_the_two_launch_path():
    banner("append_verify with K/V not 16-byte aligned")
    wl = workload(KV_BF16, 8, 2, 64, [250, 40])
    a, b = Runner(wl), Runner(wl)
    a.fill()
    b.fill()
    k, v = synth.step_kv(wl, 0, 8, "cuda")
    q = synth.queries(wl, 0, 8, "cuda")
    flat_k = torch.empty(k.numel() + 1, dtype=k.dtype, device="cuda")
    flat_v = torch.empty_like(flat_k)
    ku = flat_k[1:].view(k.shape)  # 2 bytes past a 16-byte boundary
    vu = flat_v[1:].view(v.shape)
    ku.copy_(k)
    vu.copy_(v)
    oa = a.caches[0].append_verify([0, 1], [5, 3], k, v, q, wl.hq, wl.scale)
    ob = b.caches[0].append_verify([0, 1], [5, 3], ku, vu, q, wl.hq, wl.scale)
    assert torch.equal(oa, ob)
    for s, L in ((0, 255), (1, 43)):
        xa, xb = stored(a.caches[0], s, L), stored(b.caches[0], s, L)
        assert all(np.array_equal(xa[key], xb[key]) for key in xa)
