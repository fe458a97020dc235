"""Pins of the oracle's verify attention (oracle.attention) against closed
forms, invariants and an independent library routine.

Each pin is a function of the attention callable, so the last test can plant
plausible mistakes in copies of the oracle and check that some pin catches
each of them.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A

RNG = np.random.default_rng(1234)


def rand_case(L, n, hq, hkv, d, rng=RNG):
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    return q, k, v


# ---- pins (each raises AssertionError when the attention callable is wrong) ----


def pin_weights_sum_to_one(attn):
    for window, cap in [(0, 0.0), (7, 0.0), (0, 3.0), (5, 2.0)]:
        q, k, v = rand_case(40, 5, 8, 2, 16)
        _, w = attn(q, k, v, 0.3, cap, window, return_weights=True)
        for (_, _), (_, wts) in w.items():
            assert abs(wts.sum() - 1.0) <= 1e-12
            assert np.all(wts >= 0.0)


def pin_single_visible_key(attn):
    # window 1: each row sees only its own position, so o = v at that position.
    q, k, v = rand_case(30, 5, 4, 2, 8)
    o = attn(q, k, v, 0.7, 0.0, 1)
    for i in range(5):
        p = 30 - 5 + i
        for h in range(4):
            assert np.array_equal(o[i, h], v[p, h // 2])


def pin_window_ge_context_is_full(attn):
    q, k, v = rand_case(50, 5, 6, 3, 8)
    full = attn(q, k, v, 0.5, 0.0, 0)
    for w in (50, 51, 1000):
        assert np.allclose(attn(q, k, v, 0.5, 0.0, w), full, rtol=0, atol=1e-13)
    # and a window of p keys is not full for the last row
    assert not np.allclose(attn(q, k, v, 0.5, 0.0, 49)[-1], full[-1])


def pin_zero_scale_is_mean(attn):
    L, n = 33, 4
    q, k, v = rand_case(L, n, 4, 1, 8)
    for window in (0, 6):
        o = attn(q, k, v, 0.0, 0.0, window)
        for i in range(n):
            p = L - n + i
            lo = 0 if window == 0 else max(0, p - window + 1)
            mean = v[lo: p + 1, 0].mean(axis=0)
            for h in range(4):
                assert np.allclose(o[i, h], mean, rtol=0, atol=1e-13)


def pin_two_keys_closed_form(attn):
    # q = a e_1, k_0 = e_1, k_1 = -e_1: scores s0 = a*scale, s1 = -a*scale;
    # o = sigma(s0 - s1) v0 + sigma(s1 - s0) v1 with sigma the logistic.
    d, a, scale = 4, 1.3, 0.8
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = a
    k = np.zeros((2, 1, d))
    k[0, 0, 0] = 1.0
    k[1, 0, 0] = -1.0
    v = np.array([[[1.0, 2.0, 3.0, 4.0]], [[-5.0, 0.5, 0.0, 1.0]]])
    s0, s1 = a * scale, -a * scale
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    expect = w0 * v[0, 0] + (1.0 - w0) * v[1, 0]
    assert np.allclose(attn(q, k, v, scale, 0.0, 0)[0, 0], expect, rtol=0, atol=1e-14)
    # with a soft cap c the scores become c*tanh(s/c)
    cap = 0.5
    t0, t1 = cap * math.tanh(s0 / cap), cap * math.tanh(s1 / cap)
    w0 = 1.0 / (1.0 + math.exp(t1 - t0))
    expect = w0 * v[0, 0] + (1.0 - w0) * v[1, 0]
    assert np.allclose(attn(q, k, v, scale, cap, 0)[0, 0], expect, rtol=0, atol=1e-14)


def pin_softcap_saturates(attn):
    # scores of +-100 under cap 50 become 50*tanh(+-2); a one-hot pair checks it.
    d = 2
    q = np.array([[[10.0, 0.0]]])
    k = np.array([[[10.0, 0.0]], [[-10.0, 0.0]]])  # raw scores +-100 at scale 1
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    o = attn(q, k, v, 1.0, 50.0, 0)[0, 0]
    t = 50.0 * math.tanh(2.0)
    w0 = 1.0 / (1.0 + math.exp(-2.0 * t))
    assert np.allclose(o, [w0, 1.0 - w0], rtol=0, atol=1e-14)
    del d


def pin_gqa_head_map(attn):
    # V of kv head j is the constant c_j at every position, so any query head h
    # must return c_{h // g} exactly, whatever its weights.
    L, n, hq, hkv, d = 20, 3, 12, 3, 5
    q, k, _ = rand_case(L, n, hq, hkv, d)
    consts = np.array([[1.0] * d, [-2.0] * d, [4.5] * d])
    v = np.broadcast_to(consts[None], (L, hkv, d)).copy()
    o = attn(q, k, v, 0.4, 0.0, 0)
    g = hq // hkv
    for h in range(hq):
        assert np.allclose(o[:, h], consts[h // g], rtol=0, atol=1e-14)


def pin_causal_rows(attn):
    # row i must not see the later draft rows: perturb them, earlier rows keep
    # their output, the last row changes.
    L, n = 25, 5
    q, k, v = rand_case(L, n, 4, 2, 8)
    base = attn(q, k, v, 0.5, 0.0, 0)
    k2, v2 = k.copy(), v.copy()
    k2[L - 2:] += 3.0
    v2[L - 2:] -= 7.0
    o2 = attn(q, k2, v2, 0.5, 0.0, 0)
    assert np.array_equal(o2[: n - 2], base[: n - 2])
    assert not np.allclose(o2[n - 1], base[n - 1])


def pin_matches_torch_sdpa(attn):
    # torch's scaled_dot_product_attention (CPU, fp64) with an explicit mask.
    rng = np.random.default_rng(7)
    for (L, n, hq, hkv, d, window, scale) in [(64, 5, 8, 2, 16, 0, 0.25), (90, 3, 6, 3, 8, 17, 0.4),
                                              (12, 1, 4, 4, 32, 0, 1.0), (300, 5, 32, 8, 64, 33, 0.125)]:
        q, k, v = rand_case(L, n, hq, hkv, d, rng)
        g = hq // hkv
        qt = torch.from_numpy(q).permute(1, 0, 2)  # [hq, n, d]
        kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)
        vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)
        pos = torch.arange(L - n, L)[:, None]
        key = torch.arange(L)[None, :]
        mask = key <= pos
        if window:
            mask &= (pos - key) < window
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        got = attn(q, k, v, scale, 0.0, window)
        assert np.allclose(got, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def pin_large_cap_is_no_cap(attn):
    q, k, v = rand_case(40, 5, 4, 2, 8)
    assert np.allclose(attn(q, k, v, 0.3, 1e9, 0), attn(q, k, v, 0.3, 0.0, 0), rtol=0, atol=1e-12)


def pin_single_row_is_plain_decode(attn):
    # n = 1 with no window: one query at the last position over all keys.
    L, hq, hkv, d = 37, 4, 2, 8
    q, k, v = rand_case(L, 1, hq, hkv, d)
    o = attn(q, k, v, 0.5, 0.0, 0)
    for h in range(hq):
        s = 0.5 * (k[:, h // 2] @ q[0, h])
        w = np.exp(s - s.max())
        w /= w.sum()
        assert np.allclose(o[0, h], w @ v[:, h // 2], rtol=0, atol=1e-14)


PINS = [pin_weights_sum_to_one, pin_single_visible_key, pin_window_ge_context_is_full, pin_zero_scale_is_mean,
        pin_two_keys_closed_form, pin_softcap_saturates, pin_gqa_head_map, pin_causal_rows, pin_matches_torch_sdpa,
        pin_large_cap_is_no_cap, pin_single_row_is_plain_decode]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(A.verify_attention)


def test_visible_key_count():
    assert A.visible_key_count(261, 5, 0) == 261
    assert A.visible_key_count(32773, 5, 512) == 516  # union of five 512-key windows
    assert A.visible_key_count(100, 5, 1000) == 100


# ---- planted mistakes -------------------------------------------------------------


def _mutant(kind):
    """A copy of the oracle's definition with one plausible mistake."""

    def attn(q, k, v, scale, softcap=0.0, window=0, return_weights=False):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        n, hq, d = q.shape
        L, hkv, _ = k.shape
        g = hq // hkv
        out = np.zeros((n, hq, d))
        weights = {}
        for i in range(n):
            p = L - n + i
            if kind == "row_offset":
                p = L - n + i - 1 if i > 0 else p
            lo = 0 if window == 0 else max(0, p - window + (0 if kind == "window_edge" else 1))
            hi = p + 1 if kind != "sees_future" else L
            keys = np.arange(lo, hi)
            for h in range(hq):
                kv = h % hkv if kind == "head_map" else h // g
                s = (1.0 if kind == "no_scale" else scale) * (k[keys, kv, :] @ q[i, h, :])
                if softcap > 0.0:
                    s = np.tanh(s / softcap) if kind == "cap_no_mult" else softcap * np.tanh(s / softcap)
                if kind == "max_sign":
                    e = np.exp(s + s.max())
                else:
                    e = np.exp(s - s.max())
                w = e / (e.sum() if kind != "no_norm" else 1.0)
                vv = k if kind == "k_for_v" else v
                out[i, h, :] = w @ vv[keys, kv, :]
                weights[(i, h)] = (keys, w)
        return (out, weights) if return_weights else out

    return attn


@pytest.mark.parametrize("kind", ["row_offset", "window_edge", "sees_future", "head_map", "no_scale", "cap_no_mult",
                                  "no_norm", "k_for_v"])
def test_pins_catch_planted_mistake(kind):
    bad = _mutant(kind)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bad)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the '{kind}' mistake"


# ---- the grouped arrangement (one matrix product per kv head) --------------------------


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_grouped_meets_every_pin(pin):
    pin(A.verify_attention_grouped)


@pytest.mark.parametrize("seed", range(12))
def test_grouped_equals_row_by_row(seed):
    rng = np.random.default_rng(500 + seed)
    hkv = int(rng.integers(1, 4))
    g = int(rng.integers(1, 6))
    n = int(rng.integers(1, 9))
    L = n + int(rng.integers(0, 300))
    d = int(rng.choice([8, 16, 64]))
    window = int(rng.choice([0, 1, 3, 17, 400]))
    cap = float(rng.choice([0.0, 0.7, 30.0]))
    q, k, v = rand_case(L, n, hkv * g, hkv, d, rng)
    scale = float(rng.uniform(0.05, 2.0))
    a, wa = A.verify_attention(q, k, v, scale, cap, window, return_weights=True)
    b, wb = A.verify_attention_grouped(q, k, v, scale, cap, window, return_weights=True)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    assert wa.keys() == wb.keys()
    for key in wa:
        assert np.array_equal(wa[key][0], wb[key][0])
        assert np.allclose(wa[key][1], wb[key][1], rtol=0, atol=1e-13)
