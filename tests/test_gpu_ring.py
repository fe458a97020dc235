"""GPU tests of ring caches for sliding-window layers (kv_params.ring_window),
through the C ABI.

A ring cache keeps only each sequence's last window + 8 positions, so a run
drives a plain cache and a ring cache of the same window layer with the same
inputs.  Bars:
* outputs bit-identical to the plain cache's at every step (host rollbacks;
  the call plans do not depend on block ids), and within 2e-5 with device
  rollbacks (the split is planned from length bounds);
* block tables (with released entries) and the free-block count equal the
  oracle's block-manager model driven by the same calls;
* stored bytes of every kept position equal the plain cache's;
* the pool holds n_seqs x ceil((W + 262) / 256) blocks and never runs out;
* the final outputs match the fp64 oracle (2e-3 bf16, 1e-5 fp32 and TQ3).
"""

import math

import numpy as np
import pytest
import torch

from oracle import bookkeeping as B
from parity import max_err, max_err_tq3, read_plain, read_tq3, require_gpu
from speculative_verify_attention_amd import KV_BF16, KV_EINVAL, KV_ERANGE, KV_FP32, KV_TQ3, SvattnError, synth
from speculative_verify_attention_amd.runner import Runner, ring_blocks_per_seq

pytestmark = pytest.mark.gpu

TOL = {KV_FP32: 1e-5, KV_BF16: 2e-3, KV_TQ3: 1e-5}
STEPS = 14


def banner(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def workload(fmt, hq, hkv, d, prefill, window, cap=0.0, seed=41):
    return synth.Workload("ring", hq, hkv, d, fmt, list(prefill), [5] * len(prefill), window=window, softcap=cap,
                          seed=seed, alloc_seed=0xB10C5, codec_seed=0x5EED, steps=STEPS + 2)


def plan(wl, t):
    rng = np.random.default_rng(500 + 13 * wl.seed + t)
    rows = rng.integers(1, 6, size=wl.n_seqs)
    acc = np.array([rng.integers(0, r) for r in rows])
    return rows.tolist(), acc.tolist()


def stored_from(cache, s, lo, L):
    """Stored fields of positions [lo, L) of sequence s (whole blocks read)."""
    if cache.fmt == KV_TQ3:
        return read_tq3_range(cache, s, lo, L)
    k, v = read_plain_range(cache, s, lo, L)
    it = torch.int16 if cache.fmt == KV_BF16 else torch.int32
    return {"k": k.view(it).cpu().numpy(), "v": v.view(it).cpu().numpy()}


class _Shifted:
    """A view of a cache whose table starts at block lo // 256, so the
    readback helpers (which read from position 0) see only kept blocks."""

    def __init__(self, cache, s, lo):
        self.c, self.s, self.b0 = cache, s, lo // 256
        self.num_kv_heads, self.head_dim, self.fmt, self.pool = cache.num_kv_heads, cache.head_dim, cache.fmt, cache.pool

    def block_table(self, s):
        return self.c.block_table(self.s)[self.b0:]


def read_plain_range(cache, s, lo, L):
    b0 = lo // 256
    k, v = read_plain(_Shifted(cache, s, lo), s, L - 256 * b0)
    return k[lo - 256 * b0:], v[lo - 256 * b0:]


def read_tq3_range(cache, s, lo, L):
    b0 = lo // 256
    f = read_tq3(_Shifted(cache, s, lo), s, L - 256 * b0)
    return {key: val[lo - 256 * b0:] for key, val in f.items()}


def run(wl, device_rb, fused=True, steps=STEPS):
    """Plain twin and ring cache of one window layer; returns (plain, ring,
    model, gaps, last rows/q/out)."""
    seqs = list(range(wl.n_seqs))
    layer = [(wl.window, wl.softcap)]
    a = Runner(wl, layers=layer, track=True)
    b = Runner(wl, layers=layer, track=True, ring=True, extra_blocks=(wl.n_seqs * 2 if device_rb else 0))
    ring = b.caches[0]
    assert ring.ring_window == wl.window
    model = B.KVModel(ring.params.num_blocks, wl.n_seqs, wl.max_blocks_per_seq(), alloc_seed=wl.alloc_seed,
                      ring_window=wl.window)
    a.fill()
    b.fill()
    for s, L in enumerate(wl.prefill):
        for start in range(0, L, 1 << 16):
            model.append([s], [[0] * min(1 << 16, L - start)])
    gaps, last = [], None
    for t in range(steps):
        rows, acc = plan(wl, t)
        drafts = [n - 1 for n in rows]
        rb = [d - x for d, x in zip(drafts, acc)]
        k, v = a.append_rows(t, rows)
        q = a.queries(t, rows)
        out_a = a.verify(0, rows, q)
        if fused:
            out_b = ring.append_verify(seqs, rows, k, v, q, wl.hq, wl.scale, wl.softcap, wl.window)
        else:
            ring.append(seqs, rows, k, v)
            out_b = ring.verify(seqs, rows, q, wl.hq, wl.scale, wl.softcap, wl.window)
        b.step_k.append(k.float().cpu().numpy())
        b.step_v.append(v.float().cpu().numpy())
        off = b.step_rows0
        for s, n in enumerate(rows):
            b.prov[s] = np.concatenate([b.prov[s], off + np.arange(n, dtype=np.int64)])
            off += n
        b.step_rows0 = off
        assert model.append(seqs, [[0] * n for n in rows]) == B.OK
        torch.cuda.synchronize()
        gaps.append(float((out_a - out_b).abs().max()))
        last = (rows, q, out_b)
        if not device_rb:
            for s in seqs:
                assert ring.block_table(s) == model.table[s], (t, s)
            assert ring.free_blocks() == len(model.free)
        if t == steps - 1:
            break
        a.rollback(rb)
        if device_rb:
            ring.rollback_device(seqs, drafts, torch.tensor(acc, dtype=torch.int32, device="cuda"))
            for s, r in enumerate(rb):
                if r:
                    b.prov[s] = b.prov[s][: len(b.prov[s]) - r]
        else:
            b.rollback(rb)  # moves the runner's record of positions too
            for s, r in enumerate(rb):
                if r:
                    assert model.rollback(s, r) == B.OK
    return a, b, model, gaps, last


def check(wl, device_rb, fused=True):
    a, b, model, gaps, (rows, q, out) = run(wl, device_rb, fused)
    ring = b.caches[0]
    worst = max(gaps)
    print(f"max |ring - plain| over {len(gaps)} steps: {worst:.3e}", flush=True)
    assert worst <= (2e-5 if device_rb else 0.0), gaps
    f = max_err_tq3 if wl.fmt == KV_TQ3 else max_err
    err = f(b, rows, q, out, 0, range(wl.n_seqs))
    print(f"max abs err vs oracle {err:.3e}", flush=True)
    assert err <= TOL[wl.fmt], err
    ring.sync()
    for s in range(wl.n_seqs):
        L = a.caches[0].seq_len(s)
        assert ring.seq_len(s) == L
        table = ring.block_table(s)
        kept = [i for i, x in enumerate(table) if x >= 0]
        assert len(kept) <= ring_blocks_per_seq(wl.window) + (2 if device_rb else 0)
        lo = kept[0] * 256 if kept else 0  # the first kept position
        assert lo <= max(0, L - wl.window + 1)  # everything a window can still see is kept
        assert all(x >= 0 for x in table[lo // 256: math.ceil(L / 256)])
        xa, xb = stored_from(a.caches[0], s, lo, L), stored_from(ring, s, lo, L)
        for key in xa:
            assert np.array_equal(np.asarray(xa[key]), np.asarray(xb[key])), (s, key)


# name, fmt, hq, hkv, d, prefill, window, cap
CASES = [
    ("bf16_d256_w64_cap", KV_BF16, 8, 1, 256, [300, 700, 62, 1030], 64, 50.0),
    ("bf16_d128_w512", KV_BF16, 16, 4, 128, [2000, 513, 70], 512, 0.0),
    ("fp32_d64_w1", KV_FP32, 8, 2, 64, [600, 9], 1, 0.0),
    ("tq3_d128_w96", KV_TQ3, 8, 2, 128, [900, 250, 31], 96, 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ring_equals_plain_window_layer(case):
    name, fmt, hq, hkv, d, prefill, window, cap = case
    banner(f"ring cache {name}, host rollbacks, append_verify")
    check(workload(fmt, hq, hkv, d, prefill, window, cap), device_rb=False)


@pytest.mark.parametrize("case", CASES[:2] + CASES[3:], ids=[c[0] for c in CASES[:2] + CASES[3:]])
def test_ring_with_device_rollback(case):
    name, fmt, hq, hkv, d, prefill, window, cap = case
    banner(f"ring cache {name}, device rollbacks")
    check(workload(fmt, hq, hkv, d, prefill, window, cap, seed=43), device_rb=True)


def test_ring_separate_calls():
    banner("ring cache, kv_append + spec_verify_attn")
    check(workload(KV_BF16, 8, 2, 128, [800, 100], 128), device_rb=False, fused=False)


def test_ring_errors_change_nothing():
    banner("ring cache argument errors")
    wl = workload(KV_BF16, 8, 2, 64, [1000], 100)
    b = Runner(wl, layers=[(100, 0.0)], ring=True)
    b.fill()
    c = b.caches[0]
    table, L = c.block_table(0), c.seq_len(0)
    q = synth.queries(wl, 0, 1, "cuda")
    for bad_window in (0, 101):
        with pytest.raises(SvattnError) as e:
            c.verify([0], [1], q, wl.hq, wl.scale, 0.0, bad_window)
        assert e.value.code == KV_EINVAL
    # kept from block (1000 - 107) // 256 = 3, i.e. position 768: rollback to
    # L' needs L' - 99 >= 768
    with pytest.raises(SvattnError) as e:
        c.rollback(0, 1000 - 866)
    assert e.value.code == KV_ERANGE
    with pytest.raises(SvattnError) as e:
        c.rollback_device([0], [1000 - 866], torch.zeros(1, dtype=torch.int32, device="cuda"))
    assert e.value.code == KV_ERANGE
    assert c.block_table(0) == table and c.seq_len(0) == L
    c.rollback(0, 1000 - 867)
    assert c.seq_len(0) == 867


@pytest.mark.parametrize("i", range(16))
def test_ring_sweep(i):
    """Seeded random window layers on ring caches (window 1..600, format,
    head dim, GQA group, 1..6 sequences of 8..2000 positions), host
    rollbacks for even cases and device rollbacks for odd ones."""
    rng = np.random.default_rng(7000 + i)
    fmt = (KV_FP32, KV_BF16, KV_TQ3)[i % 3]
    d = int(rng.choice([64, 128] if fmt == KV_TQ3 else [64, 128, 256]))
    hkv = int(rng.choice([1, 2]))
    g = int(rng.choice([1, 4, 8]))
    prefill = np.exp(rng.uniform(np.log(8.0), np.log(2000.0), int(rng.integers(1, 7)))).astype(int).tolist()
    window = int(rng.integers(1, 601))
    cap = float(rng.choice([0.0, 30.0]))
    banner(f"ring sweep {i}: fmt={fmt} d={d} hq={hkv * g} hkv={hkv} window={window} cap={cap} prefill={prefill}")
    check(workload(fmt, hkv * g, hkv, d, prefill, window, cap, seed=50 + i), device_rb=bool(i % 2))
