"""Host core (libsvattn_core.so, the HIP-free part of libsvattn) against the
oracle's block-manager model and codec draws, on the CPU."""

import ctypes
import os
import subprocess
import sys

import hypothesis.strategies as st
import numpy as np
import pytest
from hypothesis import settings
from hypothesis.stateful import RuleBasedStateMachine, invariant, rule

from oracle import bookkeeping as B
from oracle import splitmix, tq3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CORE = os.path.join(ROOT, "speculative_verify_attention_amd", "libsvattn_core.so")


def _core():
    if not os.path.exists(CORE):
        subprocess.run([sys.executable, "-c", "from speculative_verify_attention_amd import build; build.build_core()"],
                       cwd=ROOT, check=True)
    from speculative_verify_attention_amd import core_lib

    return core_lib()


class Core:
    def __init__(self, num_blocks, max_seqs, max_bps, alloc_seed=0, fmt=1, d=128, codec_seed=0, ring_window=0):
        from speculative_verify_attention_amd import svcore_params

        self.lib = _core()
        p = svcore_params(2, d, 256, num_blocks, max_seqs, max_bps, fmt, ring_window, alloc_seed, codec_seed)
        self.h = ctypes.c_void_p()
        rc = self.lib.svcore_create(ctypes.byref(p), ctypes.byref(self.h))
        assert rc == 0
        self.max_seqs = max_seqs

    def __del__(self):
        self.lib.svcore_destroy(self.h)

    def append(self, seqs, ns):
        a = (ctypes.c_int32 * max(1, len(seqs)))(*seqs)
        b = (ctypes.c_int32 * max(1, len(ns)))(*ns)
        return self.lib.svcore_append(self.h, len(seqs), a, b)

    def rollback(self, s, r):
        return self.lib.svcore_rollback(self.h, s, r)

    def free(self, s):
        return self.lib.svcore_seq_free(self.h, s)

    def seq_len(self, s):
        out = ctypes.c_int32()
        assert self.lib.svcore_seq_len(self.h, s, ctypes.byref(out)) == 0
        return out.value

    def table(self, s):
        buf = (ctypes.c_int32 * 4096)()
        n = ctypes.c_int32()
        assert self.lib.svcore_block_table(self.h, s, buf, 4096, ctypes.byref(n)) == 0
        return list(buf[: n.value])

    def free_blocks(self):
        out = ctypes.c_int32()
        self.lib.svcore_free_blocks(self.h, ctypes.byref(out))
        return out.value


def test_append5_rollback3_equals_append2():
    a, b = Core(16, 2, 8, alloc_seed=9), Core(16, 2, 8, alloc_seed=9)
    for c in (a, b):
        assert c.append([0], [256]) == 0
    assert a.append([0], [5]) == 0 and a.rollback(0, 3) == 0
    assert b.append([0], [2]) == 0
    assert a.seq_len(0) == b.seq_len(0) == 258
    assert a.table(0)[:2] == b.table(0)[:2]


def test_forced_failures_leave_state_unchanged():
    c = Core(3, 3, 2)
    assert c.append([0], [300]) == 0
    snap = (c.seq_len(0), c.table(0), c.free_blocks())
    assert c.append([1], [257]) == B.ENOMEM
    assert c.append([1, 2], [10, 300]) == B.ENOMEM  # all or nothing over the call
    assert c.append([0], [300]) == B.ERANGE  # table would overflow
    assert c.rollback(0, 301) == B.ERANGE
    assert c.rollback(0, -1) == B.EINVAL
    assert c.rollback(7, 1) == B.ENOSEQ
    assert c.append([5], [1]) == B.ENOSEQ
    assert c.append([1, 1], [1, 1]) == B.EINVAL
    assert c.append([1], [-1]) == B.EINVAL
    assert (c.seq_len(0), c.table(0), c.free_blocks()) == snap
    assert c.seq_len(1) == 0 and c.table(1) == []


def test_bad_params_rejected():
    from speculative_verify_attention_amd import svcore_params

    lib = _core()
    for kw in [dict(d=100), dict(bs=128), dict(nb=0), dict(fmt=7), dict(hkv=0)]:
        p = svcore_params(kw.get("hkv", 2), kw.get("d", 128), kw.get("bs", 256), kw.get("nb", 4), 2, 2,
                          kw.get("fmt", 1), 0, 0, 0)
        h = ctypes.c_void_p()
        assert lib.svcore_create(ctypes.byref(p), ctypes.byref(h)) == B.EINVAL


class CoreVsModel(RuleBasedStateMachine):
    """Random append / rollback / free sequences: the core and the oracle model
    must agree on every status code, seq_len, live table and free count."""

    def __init__(self):
        super().__init__()
        self.core = Core(24, 4, 6, alloc_seed=0xB10C5)
        self.model = B.KVModel(24, 4, 6, alloc_seed=0xB10C5)

    @rule(seqs=st.lists(st.integers(-1, 4), min_size=1, max_size=4), ns=st.lists(st.integers(-1, 700), min_size=4,
                                                                                   max_size=4))
    def append(self, seqs, ns):
        ns = ns[: len(seqs)]
        rc_core = self.core.append(seqs, ns)
        if any(n < 0 for n in ns):
            # negative counts are not representable in the model: walk the
            # entries in call order as the documented precedence says
            seen, expect = set(), None
            for sq, n in zip(seqs, ns):
                if not (0 <= sq < 4):
                    expect = B.ENOSEQ
                elif sq in seen or n < 0:
                    expect = B.EINVAL
                elif -(-(self.model.seq_len[sq] + n) // 256) > 6:
                    expect = B.ERANGE
                if expect is not None:
                    break
                seen.add(sq)
            assert rc_core == expect
            return
        rc_model = self.model.append(seqs, [[0] * n for n in ns])
        assert rc_core == rc_model

    @rule(s=st.integers(-1, 4), r=st.integers(-2, 300))
    def rollback(self, s, r):
        assert self.core.rollback(s, r) == self.model.rollback(s, r)

    @rule(s=st.integers(-1, 4))
    def free(self, s):
        assert self.core.free(s) == self.model.free_seq(s)

    @invariant()
    def agree(self):
        for s in range(4):
            assert self.core.seq_len(s) == self.model.seq_len[s]
            assert self.core.table(s) == self.model.table[s]
        assert self.core.free_blocks() == len(self.model.free)


TestCoreVsModel = CoreVsModel.TestCase
TestCoreVsModel.settings = settings(max_examples=80, stateful_step_count=40, deadline=None)


class RingCoreVsModel(CoreVsModel):
    """The same walk on ring caches (window 300): released entries (-1), the
    release-then-pop order and the rollback limit must agree too."""

    def __init__(self):
        RuleBasedStateMachine.__init__(self)
        self.core = Core(24, 4, 6, alloc_seed=0xB10C5, ring_window=300)
        self.model = B.KVModel(24, 4, 6, alloc_seed=0xB10C5, ring_window=300)


TestRingCoreVsModel = RingCoreVsModel.TestCase
TestRingCoreVsModel.settings = settings(max_examples=80, stateful_step_count=40, deadline=None)


def test_ring_worked_example_matches_model():
    c = Core(12, 1, 8, ring_window=300)
    m = B.KVModel(12, 1, 8, ring_window=300)
    for n in (600, 200, 100, 300):
        assert c.append([0], [n]) == m.append([0], [[0] * n]) == 0
        assert c.table(0) == m.table[0]
    assert c.table(0) == [-1, -1, -1, 2, 1]
    assert c.rollback(0, 134) == B.ERANGE and c.rollback(0, 133) == 0
    assert c.free(0) == 0 and c.append([0], [1]) == 0
    assert c.table(0) == [2]  # the first kept block came back first


def test_free_list_permutation_matches_model():
    for seed in (0, 1, 0xB10C5):
        c = Core(300, 1, 300, alloc_seed=seed)
        assert c.append([0], [300 * 256]) == 0
        assert c.table(0) == splitmix.free_list_order(300, seed)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_codec_constants_match_oracle(d):
    lib = _core()
    c = Core(2, 1, 2, fmt=2, d=d, codec_seed=0x5EED)
    signs = np.zeros(d, dtype=np.int8)
    s = np.zeros((d, d), dtype=np.float32)
    lev, lev16, thr = np.zeros(8), np.zeros(8), np.zeros(7)
    assert lib.svcore_codec(c.h, signs.ctypes.data, s.ctypes.data, lev.ctypes.data, lev16.ctypes.data,
                            thr.ctypes.data) == 0
    o_signs, o_s = splitmix.codec_draws(d, 0x5EED)
    oc, oc16, ot = tq3.codebook()
    assert np.array_equal(signs, o_signs)
    # both sides round the same double-precision Box-Muller value to float32;
    # allow one float32 ulp where the two libm's differ in the last double bit
    ulp = np.spacing(np.abs(o_s))
    assert np.all(np.abs(s - o_s) <= ulp)
    assert np.mean(s == o_s) > 0.999
    assert np.allclose(lev, oc, rtol=0, atol=1e-12)
    assert np.array_equal(lev16, oc16)
    assert np.allclose(thr, ot, rtol=0, atol=1e-12)


def test_half_rounding_matches_numpy():
    lib = _core()
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.uniform(0, 70000, 20000), rng.exponential(1e-5, 5000), 2.0 ** rng.uniform(-25, 16, 5000),
                         [0.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 65504.0, 65519.99, 65520.0, 2 ** -24, 2 ** -25,
                          3 * 2 ** -26, 6.1e-5]])
    out = ctypes.c_uint16()
    sat = ctypes.c_int32()
    for x in xs:
        lib.svcore_half_bits(float(x), ctypes.byref(out), ctypes.byref(sat))
        with np.errstate(over="ignore"):
            ref = np.float16(x)
        if np.isinf(ref):
            assert out.value == 0x7BFF and sat.value == 1
        else:
            assert out.value == int(ref.view(np.uint16)), x
