"""Pins of the acceptance oracle (oracle/accept.py) against closed forms and
the distributional guarantee of rejection sampling: whatever the draft
distribution, the first emitted token follows the target distribution."""

import numpy as np
import pytest
from scipy import stats

from oracle import accept as A


def test_draw_semantics():
    w = np.array([0.0, 1.0, 2.0, 0.0, 1.0])
    assert A.draw(w, 0.0) == 1  # first positive weight
    assert A.draw(w, 0.2499) == 1
    assert A.draw(w, 0.25) == 2  # cumulative must exceed u * total
    assert A.draw(w, 0.7499) == 2
    assert A.draw(w, 0.75) == 4
    assert A.draw(w, 0.999999) == 4


def test_first_argmax_ties_go_low():
    assert A.first_argmax([1.0, 3.0, 3.0, 2.0]) == 1


def test_greedy_stops_at_first_mismatch():
    V = 7
    t = np.zeros((4, V))
    t[0, 2] = t[1, 5] = t[2, 1] = t[3, 6] = 4.0
    # drafts match rows 0 and 1, then miss row 2
    acc, tok, _ = A.accept_one(t, None, [2, 5, 3], [0.5] * 4, 0.0)
    assert (acc, tok) == (2, 1)
    acc, tok, _ = A.accept_one(t, None, [2, 5, 1], [0.5] * 4, 0.0)
    assert (acc, tok) == (3, 6)  # all accepted: the bonus is row 3's argmax
    acc, tok, _ = A.accept_one(t, None, [0, 5, 1], [0.5] * 4, 0.0)
    assert (acc, tok) == (0, 2)


def test_draft_equal_to_target_is_always_accepted():
    rng = np.random.default_rng(3)
    t = rng.standard_normal((5, 50))
    for _ in range(200):
        drafts = rng.integers(0, 50, size=4)
        u = rng.random(5)
        acc, _, _ = A.accept_one(t, t[:4], drafts, u, 0.7)
        assert acc == 4


def test_point_mass_on_a_certain_token_is_accepted():
    t = np.full((2, 10), -30.0)
    t[0, 4] = 30.0  # p(4) = 1 - ~1e-25
    acc, _, _ = A.accept_one(t, None, [4], [0.999, 0.3], 1.0)
    assert acc == 1


def test_rejection_residual_excludes_overdrafted_tokens():
    # p = q except that q moves mass onto token 0: after a rejection of token
    # 0 the residual has support only where p > q
    p_logits = np.log(np.array([0.1, 0.3, 0.3, 0.3]))
    q_logits = np.log(np.array([0.4, 0.2, 0.2, 0.2]))
    t = np.stack([p_logits, p_logits])
    acc, tok, info = A.accept_one(t, q_logits[None], [0], [0.9, 0.5], 1.0)
    assert acc == 0
    r, _ = info["draw"]
    assert r[0] == 0.0 and np.allclose(r[1:], 0.1)
    assert tok == 2  # u = 0.5 of three equal weights


def _first_token_histogram(p_logits, q_logits, point_mass, trials, seed, variant=None):
    """First emitted token over many trials, with the draft token itself
    drawn from the draft distribution (or, for point masses, from a fixed
    guess distribution unrelated to p)."""
    rng = np.random.default_rng(seed)
    V = len(p_logits)
    p = A.softmax_t(p_logits, 1.0)
    q = A.softmax_t(q_logits, 1.0)
    t = np.stack([p_logits, p_logits])
    counts = np.zeros(V)
    for _ in range(trials):
        d = int(rng.choice(V, p=q))
        u = rng.random(2)
        if variant is None:
            acc, tok, _ = A.accept_one(t, None if point_mass else q_logits[None], [d], u, 1.0)
        elif variant == "inverted_ratio":  # a plausible mistake: accept iff u * p(d) < q(d)
            if u[0] * p[d] < q[d]:
                acc, tok = 1, d
            else:
                acc, tok = 0, A.draw(np.maximum(0.0, p - q), u[1])
        elif variant == "resample_from_target":  # another: redraw from p, not from (p - q)+
            if u[0] * q[d] < p[d]:
                acc, tok = 1, d
            else:
                acc, tok = 0, A.draw(p, u[1])
        counts[d if acc == 1 else tok] += 1
    return counts, p


@pytest.mark.parametrize("point_mass", [False, True])
def test_output_follows_the_target_distribution(point_mass):
    p_logits = np.log(np.array([0.05, 0.10, 0.15, 0.20, 0.20, 0.30]))
    q_logits = np.log(np.array([0.30, 0.25, 0.05, 0.05, 0.05, 0.30]))
    counts, p = _first_token_histogram(p_logits, q_logits, point_mass, 30000, 11)
    chi = stats.chisquare(counts, counts.sum() * p)
    assert chi.pvalue > 1e-4, chi


@pytest.mark.parametrize("variant", ["inverted_ratio", "resample_from_target"])
def test_planted_mistakes_break_the_distribution(variant):
    p_logits = np.log(np.array([0.05, 0.10, 0.15, 0.20, 0.20, 0.30]))
    q_logits = np.log(np.array([0.30, 0.25, 0.05, 0.05, 0.05, 0.30]))
    counts, p = _first_token_histogram(p_logits, q_logits, False, 30000, 11, variant)
    chi = stats.chisquare(counts, counts.sum() * p)
    assert chi.pvalue < 1e-6, chi


def test_batch_walks_sequences_in_order():
    rng = np.random.default_rng(5)
    n_draft = [2, 0, 3]
    V = 20
    t = rng.standard_normal((sum(n + 1 for n in n_draft), V))
    dl = rng.standard_normal((sum(n_draft), V))
    drafts = rng.integers(0, V, size=sum(n_draft))
    u = rng.random(len(t))
    acc, tok, _ = A.accept_batch(t, dl, drafts, u, n_draft, 0.8)
    a1, t1, _ = A.accept_one(t[3:4], dl[2:2], drafts[2:2], u[3:4], 0.8)
    assert (acc[1], tok[1]) == (a1, t1) == (0, A.draw(A.softmax_t(t[3], 0.8), u[3]))
