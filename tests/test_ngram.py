"""The n-gram drafter of the libraries (include/svdraft.h, host code, run
from the HIP-free core library) against the oracle's model (oracle/ngram.py),
on the CPU: the same drafts, gate and average after any stream of
observations and draft requests."""

import hypothesis.strategies as st
import pytest
from hypothesis import given, settings

from oracle.ngram import NgramModel
from speculative_verify_attention_amd import KV_EINVAL, KV_ENOSEQ, NgramDrafter, SvattnError, core_lib


def drafter(**kw):
    return NgramDrafter(lib=core_lib(), **kw)


@settings(max_examples=120, deadline=None)
@given(st.lists(st.one_of(st.tuples(st.just("observe"), st.integers(0, 2),
                                    st.lists(st.integers(0, 5), max_size=12)),
                          st.tuples(st.just("draft"), st.integers(0, 2), st.just([]))), max_size=60),
       st.integers(1, 7))
def test_library_matches_the_model(ops, max_drafts):
    d = drafter(max_seqs=3, max_drafts=max_drafts)
    models = [NgramModel(max_drafts=max_drafts) for _ in range(3)]
    for op, s, toks in ops:
        if op == "observe":
            d.observe(s, toks)
            models[s].observe(toks)
        else:
            assert d.draft(s) == models[s].draft()
        ema, on, seen = d.state(s)
        assert ema == models[s].rate  # same double-precision arithmetic, same order
        assert on == models[s].enabled() and seen == len(models[s].history)


def test_repetitive_stream_is_drafted_and_gated():
    """A periodic stream: after one period the drafts are the stream itself;
    observations that never start with the prediction (a fresh token, then a
    known one, so a prediction keeps existing) close the gate on the 7th."""
    d = drafter(max_seqs=1)
    period = [3, 1, 4, 1, 5, 9, 2, 6]
    d.observe(0, period * 2)
    for step in range(10):
        drafts = d.draft(0)
        pos = 16 + 4 * step
        assert drafts == [period[(pos + i) % 8] for i in range(4)]
        d.observe(0, drafts)
    assert d.state(0)[0] == 1.0
    for i in range(7):
        assert d.draft(0) != []
        d.observe(0, [100 + i, period[i]])
    assert d.state(0)[1] is False and d.draft(0) == []


def test_batch_calls_equal_single_calls():
    a, b = drafter(max_seqs=4), drafter(max_seqs=4)
    streams = [[1, 2, 1, 2, 1], [7, 7, 7], [5, 6, 7, 5, 6], [9]]
    a.observe_batch([0, 1, 2, 3], streams)
    for s, t in enumerate(streams):
        b.observe(s, t)
    assert a.draft_batch([3, 0, 2, 1]) == [b.draft(3), b.draft(0), b.draft(2), b.draft(1)]


def test_errors():
    with pytest.raises(SvattnError):
        drafter(max_seqs=1, max_drafts=8)
    with pytest.raises(SvattnError):
        drafter(max_seqs=1, ema_tau=0.0)
    d = drafter(max_seqs=2)
    with pytest.raises(SvattnError) as e:
        d.observe(2, [1])
    assert e.value.code == KV_ENOSEQ
    with pytest.raises(SvattnError) as e:
        d.observe(0, [1, -2])
    assert e.value.code == KV_EINVAL
    with pytest.raises(SvattnError):
        d.observe_batch([0, 1], [[1, 2], [3, -1]])
    assert d.state(0)[2] == 0 and d.state(1)[2] == 0  # nothing observed by the failed calls
    d.observe(0, [1, 2, 1])
    d.reset(0)
    assert d.state(0) == (1.0, True, 0) and d.draft(0) == []
