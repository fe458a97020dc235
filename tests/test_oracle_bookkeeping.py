"""Pins of the oracle's block-manager model (oracle.bookkeeping): the pages'
rollback rule (append 5 then roll back 3 equals appending 2), the 256-token
block invariant, conservation of blocks, and all-or-nothing failures."""

import math
import random

import hypothesis.strategies as st
from hypothesis import given, settings

from oracle import bookkeeping as B


def state(m, s):
    return m.seq_len[s], m.live_table(s), m.contents(s)


def test_append5_rollback3_equals_append2():
    a = B.KVModel(16, 2, 8, alloc_seed=3)
    b = B.KVModel(16, 2, 8, alloc_seed=3)
    for m in (a, b):
        assert m.append([0], [list(range(256))]) == B.OK
    assert a.append([0], [["d0", "d1", "d2", "d3", "d4"]]) == B.OK
    assert a.rollback(0, 3) == B.OK
    assert b.append([0], [["d0", "d1"]]) == B.OK
    assert state(a, 0) == state(b, 0)
    assert a.seq_len[0] == 258


def test_rollback_keeps_blocks_and_next_append_overwrites():
    m = B.KVModel(8, 1, 8)
    m.append([0], [list(range(300))])
    owned = list(m.table[0])
    m.rollback(0, 100)
    assert m.table[0] == owned and m.live_table(0) == owned[:1]
    m.append([0], [["x"] * 10])
    assert m.table[0] == owned
    assert m.contents(0)[200:210] == ["x"] * 10 and len(m.contents(0)) == 210


def test_errors_leave_state_unchanged():
    m = B.KVModel(3, 2, 2)
    assert m.append([0], [[1] * 300]) == B.OK  # 2 blocks
    snap = (list(m.free), [list(t) for t in m.table], list(m.seq_len))
    assert m.append([1], [[1] * 257]) == B.ENOMEM  # needs 2, 1 free
    assert (list(m.free), [list(t) for t in m.table], list(m.seq_len)) == snap
    assert m.append([0, 1], [[1] * 10, [1] * 257]) == B.ENOMEM  # all-or-nothing over the call
    assert (list(m.free), [list(t) for t in m.table], list(m.seq_len)) == snap
    m2 = B.KVModel(3, 2, 2)
    m2.append([0], [[1] * 300])
    assert m2.append([0], [[1] * 300]) == B.ERANGE  # would need 3 > max 2
    assert m2.rollback(0, 301) == B.ERANGE
    assert m2.rollback(0, -1) == B.EINVAL
    assert m2.rollback(5, 1) == B.ENOSEQ
    assert m2.append([0, 0], [[1], [1]]) == B.EINVAL
    assert (list(m2.free), [list(t) for t in m2.table], list(m2.seq_len)) == snap


def test_free_returns_first_owned_block_first():
    m = B.KVModel(10, 2, 5, alloc_seed=11)
    order = list(m.free)
    m.append([0], [[0] * 600])  # 3 blocks
    assert m.table[0] == order[:3]
    m.free_seq(0)
    assert m.free[:3] == order[:3]
    m.append([1], [[0] * 10])
    assert m.table[1] == [order[0]]


@settings(max_examples=60, deadline=None)
@given(st.lists(st.tuples(st.sampled_from(["append", "rollback", "free"]), st.integers(0, 3), st.integers(0, 600)),
                max_size=40), st.sampled_from([0, 1, 300]))
def test_invariants_under_random_ops(ops, ring):
    m = B.KVModel(12, 4, 8, alloc_seed=5, ring_window=ring)
    for op, s, n in ops:
        if op == "append":
            m.append([s], [[(s, i) for i in range(n)]])
        elif op == "rollback":
            m.rollback(s, n % 50)
        else:
            m.free_seq(s)
        owned = [b for t in m.table for b in t if b >= 0]
        assert len(owned) == len(set(owned))
        assert sorted(owned + m.free) == list(range(12))
        for q in range(4):
            assert len(m.table[q]) >= math.ceil(m.seq_len[q] / 256)
            assert len(m.live_table(q)) == math.ceil(m.seq_len[q] / 256)
            # every position a window can still see has its block
            lo = max(0, m.seq_len[q] - ring + 1) if ring else 0
            assert m.first_position(q) <= lo or m.seq_len[q] == 0
            assert all(b >= 0 for b in m.table[q][lo // 256: math.ceil(m.seq_len[q] / 256)])


# ---- ring caches for window layers ---------------------------------------------------


def test_ring_worked_example():
    """W = 300, one sequence, identity free list; every step worked by hand:
    the first kept block is max(0, L - 8 - 300 + 1) // 256."""
    m = B.KVModel(12, 1, 8, ring_window=300)
    assert m.append([0], [[0] * 600]) == B.OK  # keep from (600-307)//256 = 1: index 0 never held
    assert m.table[0] == [-1, 0, 1] and m.first[0] == 1 and m.free[:2] == [2, 3]
    assert m.append([0], [[0] * 200]) == B.OK  # L 800, keep 1; one new block
    assert m.table[0] == [-1, 0, 1, 2]
    assert m.append([0], [[0] * 100]) == B.OK  # L 900, keep 2: index 1 (block 0) released
    assert m.table[0] == [-1, -1, 1, 2] and m.free[:2] == [0, 3]
    assert m.append([0], [[0] * 300]) == B.OK  # L 1200, keep 3: release block 1, then pop it again
    assert m.table[0] == [-1, -1, -1, 2, 1] and m.free[:2] == [0, 3]
    # a later window must not reach below position 768: max(0, L' - 299) >= 768
    assert m.rollback(0, 134) == B.ERANGE
    assert m.rollback(0, 133) == B.OK and m.seq_len[0] == 1067
    assert m.free_seq(0) == B.OK
    assert m.free[:2] == [2, 1]  # the kept blocks, first-kept first


def test_ring_memory_stays_bounded():
    """Decode-like steps (append 1 + k, roll back up to k) over 6000 positions
    with W = 512: never more than 4 blocks kept, and a plain cache of the
    same steps agrees on lengths and contents."""
    rng = random.Random(7)
    ring = B.KVModel(8, 1, 64, ring_window=512)
    plain = B.KVModel(64, 1, 64)
    step = 0
    while ring.seq_len[0] < 6000:
        n = rng.randint(1, 5)
        items = [(step, i) for i in range(n)]
        assert ring.append([0], [items]) == B.OK
        assert plain.append([0], [items]) == B.OK
        assert len(ring.kept_blocks(0)) <= 4
        r = rng.randint(0, n - 1)
        assert ring.rollback(0, r) == B.OK and plain.rollback(0, r) == B.OK
        step += 1
    assert ring.seq_len[0] == plain.seq_len[0]
    assert ring.contents(0) == plain.contents(0)
    lo = ring.first_position(0)
    assert lo <= ring.seq_len[0] - 512 - 8
    assert all(b >= 0 for b in ring.table[0][lo // 256:])


def test_ring_release_makes_room_in_the_same_call():
    """A pool of exactly the kept-block bound never runs out."""
    m = B.KVModel(3, 1, 40, ring_window=200)
    for _ in range(200):
        assert m.append([0], [[0] * 37]) == B.OK
    assert len(m.kept_blocks(0)) <= 3 and len(m.free) + len(m.kept_blocks(0)) == 3
