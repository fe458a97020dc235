"""GPU parity of the compressed (TQ3) cache path against the fp64 oracle.

* codec constants: the library's rotation signs, QJL matrix, Lloyd-Max levels
  and thresholds equal the oracle's own draws and solution;
* encoded fields (codes, sign bits, fp16 norms): bit-exact, except values
  within 1e-5 of a decision boundary, which are counted (<= 0.01%);
* attention output: max abs error <= 1e-5 against the oracle's attention on
  its own decoding of the same fp32 source rows.
"""

import math

import numpy as np
import pytest
import torch

from oracle import tq3
from parity import (compare_tq3_fields, max_err_tq3, oracle_codec, read_tq3, require_gpu, unpack_records)
from speculative_verify_attention_amd import KV_TQ3, KVCache, synth
from speculative_verify_attention_amd.runner import Runner

pytestmark = pytest.mark.gpu

TOL = 1e-5
MAX_EXCLUDED = 1e-4  # fraction of fields allowed in the boundary band


def banner(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("d", [64, 128, 256])
def test_codec_constants(d):
    banner(f"tq3 codec constants d={d}")
    c = KVCache(2, d, 4, 1, 2, KV_TQ3, codec_seed=0x5EED)
    signs, s, lev, lev16, thr = c.codec()
    pi, o_s, oc, oc16, ot, o_signs = oracle_codec(d, 0x5EED)
    assert np.array_equal(signs, o_signs)
    assert np.all(np.abs(s - o_s) <= np.spacing(np.abs(o_s)))
    assert np.allclose(lev, oc, rtol=0, atol=1e-12)
    assert np.array_equal(lev16, oc16)
    assert np.allclose(thr, ot, rtol=0, atol=1e-12)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("is_key", [True, False])
def test_encode_fields(d, is_key):
    banner(f"tq3 encode fields d={d} key={is_key}")
    c = KVCache(1, d, 4, 1, 2, KV_TQ3, codec_seed=0x5EED)
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + d + is_key)
    x = torch.randn((20000, d), generator=g, device="cuda")
    x[0] = 0.0  # zero vector
    x[1] *= 1e4  # large norm (saturates fp16 at 65504)
    x[2] *= 1e-7  # tiny norm (fp16 subnormal)
    x[3, :] = 1.0  # all-equal coordinates
    rec = c.encode(x, is_key)
    torch.cuda.synchronize()
    got = unpack_records(rec.cpu().numpy(), d, is_key)
    pi, s_mat, _, c16, t, _ = oracle_codec(d, 0x5EED)
    ora = tq3.encode_batch(x.cpu().numpy().astype(np.float64), is_key, pi, s_mat, c16, t)
    mism, excl, total = compare_tq3_fields(got, ora, is_key)
    print(f"fields: mismatches {mism}, boundary-excluded {excl} of {total}", flush=True)
    assert mism == 0
    assert excl <= MAX_EXCLUDED * total
    assert got["n16"][1] == 65504.0
    # the saturated norm of x[1] is recorded in the status word; vectors
    # without one leave it clear
    assert c.read_status(clear=True) & 1
    assert c.read_status() == 0
    c.encode(x[2:], is_key)
    assert c.read_status() == 0


def tq3_workload(name, prefill, rows, d=128, hq=32, hkv=8, window=0, cap=0.0, seed=7):
    return synth.Workload(name, hq, hkv, d, KV_TQ3, prefill, rows, window=window, softcap=cap, seed=seed,
                          codec_seed=0x5EED, alloc_seed=23)


def test_pool_fields_after_append():
    banner("tq3 pool fields after append")
    wl = tq3_workload("tq3_fields", [300, 33, 7], [5, 2, 1], hkv=2, hq=8)
    r = Runner(wl, track=True)
    r.fill()
    r.step(0)
    torch.cuda.synchronize()
    pi, s_mat, _, c16, t, _ = oracle_codec(wl.d, wl.codec_seed)
    for s in range(wl.n_seqs):
        L = r.caches[0].seq_len(s)
        got = read_tq3(r.caches[0], s, L)
        k, v = r.logical_kv(s)
        ko = tq3.encode_batch(k.reshape(-1, wl.d), True, pi, s_mat, c16, t)
        vo = tq3.encode_batch(v.reshape(-1, wl.d), False, pi, s_mat, c16, t)
        gk = {"code": got["kcode"].reshape(-1, wl.d), "bits": got["kbit"].reshape(-1, wl.d),
              "n16": got["kn16"].reshape(-1), "g16": got["kg16"].reshape(-1)}
        gv = {"code": got["vcode"].reshape(-1, wl.d), "n16": got["vn16"].reshape(-1)}
        mk, ek, tk = compare_tq3_fields(gk, ko, True)
        mv, ev, tv = compare_tq3_fields(gv, vo, False)
        assert mk == 0 and mv == 0, (s, mk, mv)
        assert ek <= MAX_EXCLUDED * tk and ev <= MAX_EXCLUDED * tv


def test_append5_rollback3_equals_append2():
    banner("tq3 append-5/rollback-3 vs append-2")
    wl = tq3_workload("tq3_rb", [250], [5], hkv=2, hq=8)
    a, b = Runner(wl), Runner(wl)
    a.fill()
    b.fill()
    k, v = synth.step_kv(wl, 0, 5, "cuda")
    a.caches[0].append([0], [5], k, v)
    a.caches[0].rollback(0, 3)
    b.caches[0].append([0], [2], k[:2].contiguous(), v[:2].contiguous())
    ca, cb = a.caches[0], b.caches[0]
    assert ca.seq_len(0) == cb.seq_len(0) == 252
    fa, fb = read_tq3(ca, 0, 252), read_tq3(cb, 0, 252)
    for key in fa:
        assert np.array_equal(fa[key], fb[key]), key
    q = synth.queries(wl, 0, 2, "cuda")
    oa = ca.verify([0], [2], q, wl.hq, wl.scale)
    ob = cb.verify([0], [2], q, wl.hq, wl.scale)
    assert torch.equal(oa, ob)


def run_and_check(wl, seqs=None, layers=None, scale_q=1.0, fused=False, ring=False):
    r = Runner(wl, layers=layers, track=True, ring=ring)
    r.fill()
    rows, q, outs = r.step(0, scale_q, fused=fused)
    torch.cuda.synchronize()
    worst = 0.0
    for li, out in enumerate(outs):
        for s in (seqs if seqs is not None else range(wl.n_seqs)):
            e = max_err_tq3(r, rows, q, out, li, [s])
            print(f"  layer {li} sequence {s}: max abs err {e:.3e}", flush=True)
            worst = max(worst, e)
    return worst


def test_tq3_512():
    banner("tq3 4x512, kv_append_verify (the bench's launch), every sequence")
    err = run_and_check(synth.tq3_long(512), fused=True)
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL, err


@pytest.mark.timeout(900)
def test_tq3_40000_every_sequence():
    banner("tq3 4x40000, kv_append_verify (the bench's launch), every sequence")
    err = run_and_check(synth.tq3_long(40000), fused=True)
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL, err


@pytest.mark.timeout(1200)
def test_tq3_100000_every_sequence():
    banner("tq3 4x100000, kv_append_verify (the bench's launch), every sequence")
    err = run_and_check(synth.tq3_long(100000), fused=True)
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL, err


@pytest.mark.timeout(900)
def test_gemma_tq3_full_fused_ring():
    # the Gemma-shaped workload on a compressed cache at its bench size and
    # launch: 8 x 32K, d = 256, 5 rows x 8 heads = 40 columns (two head
    # slices), window layer on a ring cache + full layer, soft cap 50
    banner("gemma tq3 8x32768, window layer on a ring cache + full layer, kv_append_verify, every sequence")
    wl = synth.gemma_interleaved(fmt=KV_TQ3)
    err = run_and_check(wl, layers=[(512, 50.0), (0, 50.0)], fused=True, ring=True)
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL, err


@pytest.mark.timeout(900)
@pytest.mark.parametrize("scale_q,cap", [(3.0, 0.0), (2.5, 5.0)], ids=["sharp", "sharp_softcap"])
def test_tq3_long_sharp_scores(scale_q, cap):
    # every row sees more than 65,536 keys, with peaked scores: rounding
    # errors of the score products no longer average out over many
    # near-equal weights
    banner(f"tq3 1x70000, scale_q {scale_q}, softcap {cap}")
    wl = tq3_workload("tq3_sharp", [70000], [5], cap=cap, seed=int(10 * scale_q + cap))
    err = run_and_check(wl, scale_q=scale_q, fused=True)
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL, err


EDGE = [
    # name, hq, hkv, d, prefill, rows, window, cap, scale_q
    ("d64", 8, 2, 64, [700, 40], [5, 3], 0, 0.0, 1.0),
    ("plain_decode", 8, 2, 128, [1000, 5], [1, 1], 0, 0.0, 1.0),
    ("max_rows", 8, 2, 128, [300], [8], 0, 0.0, 1.0),
    ("two_column_groups", 24, 2, 128, [900, 60], [5, 4], 0, 0.0, 1.0),
    ("window", 8, 1, 128, [2000, 100], [5, 2], 512, 0.0, 1.0),
    ("softcap", 8, 2, 128, [800], [5], 0, 5.0, 3.0),
    ("short", 4, 1, 64, [0, 3], [5, 1], 0, 0.0, 1.0),
    ("ragged_many", 8, 2, 128, [int(x) for x in np.linspace(1, 2000, 40)], [3] * 40, 0, 0.0, 1.0),
    # more than 64 sequences in a launch (two lanes' worth of per-sequence
    # fields) and more than one launch
    ("many_seqs", 8, 2, 64, [int(x) for x in np.linspace(1, 700, 140)], [2] * 140, 0, 0.0, 1.0),
    ("single_pair_long", 8, 1, 128, [30000], [5], 0, 0.0, 1.0),
    # more than 64 query columns per kv head: head slices
    ("head_slices_g16", 32, 2, 128, [1500, 90], [5, 3], 0, 0.0, 1.0),
    ("head_slices_g64", 64, 1, 64, [600], [8], 0, 0.0, 2.0),
    # many query vectors (60 sequences x 1..5 rows x 32 heads, about 5,800)
    # for value-dependent rounding cases such as exact fp16 ties
    ("stress_short", 32, 8, 128, np.random.default_rng(60).integers(1, 1500, size=60).tolist(),
     np.random.default_rng(61).integers(1, 6, size=60).tolist(), 0, 0.0, 1.0),
    # head_dim 256: one 32-column group per workgroup, wider groups in head
    # slices (5 rows x 8 heads = 40 columns: two slices of 4 heads)
    ("d256_slices", 8, 1, 256, [1500, 90], [5, 3], 0, 0.0, 1.0),
    ("d256_one_group", 4, 1, 256, [3000], [8], 0, 0.0, 1.0),
    ("d256_window_softcap", 8, 2, 256, [2500, 300], [4, 2], 512, 30.0, 2.0),
    ("d256_short", 2, 1, 256, [0, 3], [5, 1], 0, 0.0, 1.0),
    ("d256_ragged", 16, 2, 256, [int(x) for x in np.linspace(1, 2000, 24)], [3] * 24, 0, 0.0, 1.0),
    ("d256_long_pair", 8, 1, 256, [20000], [4], 0, 0.0, 1.0),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge(case):
    name, hq, hkv, d, prefill, rows, window, cap, scale_q = case
    banner(f"tq3 edge {name}")
    wl = tq3_workload(name, prefill, rows, d=d, hq=hq, hkv=hkv, window=window, cap=cap, seed=len(name))
    err = run_and_check(wl, scale_q=scale_q)
    assert err <= TOL, err
