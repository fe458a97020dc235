"""The verify-call planner on the host-only core (svcore_plan_verify): for
random batches of lengths, row counts, head groupings, windows, pending
device rollbacks and fused appends, the plan is accepted exactly when the
arguments are valid, and the library's own invariant check (launch and
chunk tables, partial slots, row offsets, workspace bytes) passes; the
byte counts and chunk counts are also re-derived here from their
definitions.  AX Engine page, "Core Technical Architecture & Methods" (1 + k
rows per sequence verified against its cache); SwiftLM page, long-context
passage (one long pair split over many workgroups, partials merged)."""

import ctypes
import math

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

KV_OK, KV_EINVAL, KV_ERANGE, KV_ENOSEQ = 0, -1, -3, -4
PLAN_BROKEN = -5


def lib():
    from speculative_verify_attention_amd import core_lib

    return core_lib()


class HostCore:
    def __init__(self, hkv, d, fmt, lens, ring_window=0):
        from speculative_verify_attention_amd import svcore_params

        self.lib = lib()
        self.hkv, self.d, self.fmt = hkv, d, fmt
        max_bps = max(1, max(math.ceil((L + 8) / 256) for L in lens) + 1)
        nb = sum(math.ceil((L + 8) / 256) + 1 for L in lens)
        p = svcore_params(hkv, d, 256, nb, len(lens), max_bps, fmt, ring_window, 0, 0)
        self.h = ctypes.c_void_p()
        assert self.lib.svcore_create(ctypes.byref(p), ctypes.byref(self.h)) == 0
        seqs = [i for i, L in enumerate(lens) if L > 0]
        if seqs:
            a = (ctypes.c_int32 * len(seqs))(*seqs)
            b = (ctypes.c_int32 * len(seqs))(*[lens[i] for i in seqs])
            assert self.lib.svcore_append(self.h, len(seqs), a, b) == 0

    def close(self):
        self.lib.svcore_destroy(self.h)

    def plan(self, seqs, rows, hq, window=0, pending=None, fused=False):
        n = len(seqs)
        a = (ctypes.c_int32 * n)(*seqs)
        r = (ctypes.c_int32 * n)(*rows)
        summ = (ctypes.c_int64 * 7)()
        ks = (ctypes.c_int32 * n)()
        pend = None if pending is None else (ctypes.c_int32 * len(pending))(*pending)
        rc = self.lib.svcore_plan_verify(self.h, n, a, r, hq, window, pend, 1 if fused else 0, summ, ks)
        err = self.lib.svcore_last_error(self.h)
        return rc, list(summ), list(ks), (err or b"").decode()


def tile_keys(fmt, d):
    return 32 * max(1, 128 // d) if fmt == 1 else 32


def align(x):
    return -(-x // 256) * 256


def expected_valid(lens, seqs, rows, g, window, pending, fused):
    if min(rows) < 1 or max(rows) > 8:
        return False
    for s, n in zip(seqs, rows):
        up = lens[s] + (n if fused else 0)
        low = up - (pending[s] if pending else 0)
        if n > low:
            return False
    return True


@st.composite
def batches(draw):
    hkv = draw(st.sampled_from([1, 2, 8]))
    d = draw(st.sampled_from([64, 128, 256]))
    fmt = draw(st.sampled_from([0, 1, 2]))
    g = draw(st.sampled_from([1, 2, 4, 8, 12, 13, 16, 64]))
    n = draw(st.integers(1, 300))
    long_ = draw(st.booleans())
    hi = 120000 if long_ else 3000
    lens = draw(st.lists(st.integers(0, hi), min_size=n, max_size=n))
    k = draw(st.integers(1, n))
    seqs = draw(st.permutations(list(range(n))))[:k]
    rows = draw(st.lists(st.integers(1, 8), min_size=k, max_size=k))
    window = draw(st.sampled_from([0, 0, 1, 7, 512, 4096]))
    pending = draw(st.one_of(st.none(), st.lists(st.integers(0, 4), min_size=n, max_size=n)))
    fused = draw(st.booleans())
    return hkv, d, fmt, g, lens, seqs, rows, window, pending, fused


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(batches())
def test_plans_hold_their_invariants(b):
    hkv, d, fmt, g, lens, seqs, rows, window, pending, fused = b
    c = HostCore(hkv, d, fmt, lens)
    try:
        rc, summ, ks, err = c.plan(seqs, rows, hkv * g, window, pending, fused)
        assert rc != PLAN_BROKEN, err
        valid = expected_valid(lens, seqs, rows, g, window, pending, fused)
        assert (rc == KV_OK) == valid, (rc, err)
        if rc != KV_OK:
            assert rc in (KV_EINVAL, KV_ERANGE)
            return
        nct, launches, slots, total, part, qb, hs = summ
        # head slices: the fewest equal slices of the group whose columns fit
        # the kernel's workgroup (64 columns; 32 for the compressed format at
        # d = 256, whose workgroup holds one column group)
        cap = 32 if fmt == 2 and d == 256 else 64
        hs_want = min(h for h in range(1, g + 1) if g % h == 0 and max(rows) * (g // h) <= cap)
        assert hs == hs_want
        assert nct == (2 if max(rows) * (g // hs) > 32 else 1)
        assert launches == math.ceil(len(seqs) / 128)
        tk = tile_keys(fmt, d)
        n_tiles = []
        for s, n in zip(seqs, rows):
            up = lens[s] + (n if fused else 0)
            low = up - (pending[s] if pending else 0)
            klo = max(0, low - n - window + 1) if window > 0 else 0
            n_tiles.append(-(-up // tk) - klo // tk)
        for t, k in zip(n_tiles, ks):
            assert 1 <= k <= t
        assert slots == sum(k * hkv for k in ks)
        assert part == align(hs * slots * 32 * nct * (2 + d) * 4)
        assert qb == (align(sum(rows) * hkv * g * d * 4) if fmt == 2 else 0)
        assert total == part + 2 * qb
    finally:
        c.close()


def test_uniform_long_batch_fills_one_round():
    # 4 x 100,005 keys, 8 kv heads, compressed cache: 3,126 tiles per pair,
    # at most ceil(100,032 / 256) = 391 tiles per workgroup, so 8 chunks per
    # pair and 4 x 8 x 8 = 256 workgroups, one per compute unit
    c = HostCore(8, 128, 2, [100000] * 4)
    try:
        rc, summ, ks, err = c.plan([0, 1, 2, 3], [5] * 4, 32, fused=True)
        assert rc == KV_OK, err
        assert ks == [8] * 4 and summ[2] == 256 and summ[0] == 1
    finally:
        c.close()


def test_ragged_batch_gets_four_rounds():
    # lengths far apart: four times as many, smaller chunks
    lens = [100000, 512, 700, 40000]
    c = HostCore(8, 128, 1, lens)
    try:
        rc, summ, ks, err = c.plan([0, 1, 2, 3], [5, 1, 2, 3], 32)
        assert rc == KV_OK, err
        tiles = [-(-L // tile_keys(1, 128)) for L in lens]
        per_wg = max(4, -(-sum(t * 8 for t in tiles) // 1024))
        for t, k in zip(tiles, ks):
            k0 = max(1, -(-t // per_wg))
            cs = -(-t // k0)
            assert k == -(-t // cs)
    finally:
        c.close()


@pytest.mark.parametrize("n", [127, 128, 129, 257])
def test_launch_boundaries(n):
    c = HostCore(2, 64, 0, [300] * n)
    try:
        rc, summ, ks, err = c.plan(list(range(n)), [3] * n, 8)
        assert rc == KV_OK, err
        assert summ[1] == math.ceil(n / 128)
    finally:
        c.close()


@pytest.mark.parametrize(
    "hkv,hq,rows,hs,nct",
    [
        (2, 32, [4, 4], 1, 2),   # 4 x 16 = 64 columns: one pass
        (2, 32, [5, 4], 2, 2),   # 5 x 16 = 80: two slices of 8 heads (40 columns)
        (1, 12, [8], 2, 2),      # 8 x 12 = 96: two slices of 6 heads (48)
        (1, 64, [8, 1], 8, 2),   # 8 x 64 = 512: eight slices of 8 heads (64)
        (1, 64, [3], 4, 2),      # 3 x 64 = 192: four slices of 16 heads (48)
        (1, 7, [8], 1, 2),       # 8 x 7 = 56: fits
        (1, 14, [8], 2, 2),      # 8 x 14 = 112: two slices of 7 (56)
        (1, 13, [5], 13, 1),     # a prime group of 13 x 5 rows = 65: one head per slice
    ],
)
def test_head_slices(hkv, hq, rows, hs, nct):
    c = HostCore(hkv, 128, 1, [100] * len(rows))
    try:
        rc, summ, _, err = c.plan(list(range(len(rows))), rows, hq)
        assert rc == KV_OK, err
        assert summ[6] == hs and summ[0] == nct
        assert summ[4] == align(hs * summ[2] * 32 * nct * (2 + 128) * 4)
    finally:
        c.close()


@pytest.mark.parametrize(
    "hq,rows,hs",
    [
        (8, [4], 1),    # 4 x 8 = 32 columns: one group
        (8, [5], 2),    # 5 x 8 = 40: two slices of 4 heads (20)
        (16, [8], 4),   # 8 x 16 = 128: four slices of 4 heads (32)
        (4, [8, 3], 1),  # 8 x 4 = 32: fits
    ],
)
def test_head_slices_compressed_d256(hq, rows, hs):
    # the compressed format at d = 256 runs one 32-column group per workgroup
    c = HostCore(1, 256, 2, [100] * len(rows))
    try:
        rc, summ, _, err = c.plan(list(range(len(rows))), rows, hq)
        assert rc == KV_OK, err
        assert summ[6] == hs and summ[0] == 1
    finally:
        c.close()
