"""Pins of the n-gram drafter model (oracle/ngram.py): hand-worked drafts,
the trigram -> bigram fallback, frequency before recency, the draft cap, and
the acceptance gate against its closed form."""

import math

from oracle.ngram import NgramModel


def model_after(tokens, **kw):
    m = NgramModel(**kw)
    m.observe(tokens)
    return m


def test_worked_example_ties_go_to_the_latest():
    # (5, 6) was followed by 7 (index 2) and by 8 (index 5): one each, 8 is newer
    m = model_after([5, 6, 7, 5, 6, 8, 5, 6])
    # then (6, 8) -> 5, (8, 5) -> 6, (5, 6) -> 8 again
    assert m.draft() == [8, 5, 6, 8]


def test_bigram_fallback():
    m = model_after([1, 2, 3, 9, 2])
    # (9, 2) unseen -> bigram 2 -> 3; (2, 3) -> 9; (3, 9) -> 2; (9, 2) unseen -> bigram 2 -> 3
    assert m.draft() == [3, 9, 2, 3]


def test_frequency_beats_recency():
    m = model_after([1, 2, 3, 1, 2, 3, 1, 2, 4, 1, 2])
    assert m.draft()[0] == 3  # (1, 2) -> 3 twice, -> 4 once (later)


def test_no_evidence_no_draft():
    assert model_after([]).draft() == []
    assert model_after([7]).draft() == []
    assert model_after([1, 2]).draft() == []  # nothing ever followed 2


def test_cap():
    m = model_after([4] * 10, max_drafts=2)
    assert m.draft() == [4, 4]
    assert model_after([4] * 10, max_drafts=7).draft() == [4] * 7


def test_gate_closes_after_seven_misses_and_reopens():
    """rate starts at 1; each fully missed prediction multiplies it by 0.9, so
    the gate (rate >= 0.5) closes on the 7th miss (0.9^7 = 0.478); matched
    predictions, scored while closed too, pull it back as 1 - (1 - r) 0.9^m."""
    m = model_after([1, 2, 1, 2, 1, 2])
    expect = 1.0
    for i in range(1, 8):
        d = m.draft()
        assert (len(d) > 0) == (i < 8)  # offered before the update of this step
        m.observe([99, 98])  # never what was predicted
        m.observe([1, 2, 1, 2])  # keep the tables repetitive; nothing pending: no update
        expect = 0.9 * expect
        assert math.isclose(m.rate, expect, rel_tol=0, abs_tol=1e-15)
        assert m.enabled() == (expect >= 0.5)
    assert not m.enabled() and m.draft() == []
    r = m.rate
    for k in range(1, 10):
        pred = m.predict()
        m.draft()
        m.observe(pred)  # the text follows the prediction exactly
        assert math.isclose(m.rate, 1 - (1 - r) * 0.9 ** k, rel_tol=0, abs_tol=1e-12)
        if m.enabled():
            break
    assert m.enabled() and k == 1 + math.floor(math.log((1 - 0.5) / (1 - r)) / math.log(0.9))


def test_partial_match_scores_the_common_prefix():
    m = model_after([1, 2, 3, 1, 2, 3, 1, 2])
    assert m.draft() == [3, 1, 2, 3]
    m.observe([3, 1, 5])  # two of four
    assert math.isclose(m.rate, 0.9 + 0.1 * 0.5)


def test_planted_mistake_oldest_on_ties_fails():
    class Oldest(NgramModel):
        @staticmethod
        def _best(conts):
            return max(conts.items(), key=lambda kv: (kv[1][0], -kv[1][1]))[0]

    m = Oldest()
    m.observe([5, 6, 7, 5, 6, 8, 5, 6])
    assert m.draft() != [8, 5, 6, 8]
