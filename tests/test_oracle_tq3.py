"""Pins of the oracle's compressed-cache codec (oracle.tq3) and of the seeded
draws it uses (oracle.splitmix): published tables, closed forms, library
routines, brute force and statistical invariants."""

import math

import numpy as np
import pytest
import scipy.linalg

from oracle import splitmix, tq3


@pytest.fixture(scope="module")
def cb():
    return tq3.codebook()


# ---- Lloyd-Max codebook ------------------------------------------------------------


def test_lloyd_max_matches_max_1960(golden):
    c, t, mse, resid = tq3.lloyd_max_gaussian()
    rows = golden("lloyd_max_gaussian_8.txt")
    outs = [float(r[2]) for r in rows if r[0] == "output"]
    thrs = [float(r[2]) for r in rows if r[0] == "threshold"]
    mse_pub = [float(r[2]) for r in rows if r[0] == "mse"][0]
    # the table prints 4 significant figures: agree to half a unit in the last place
    for got, pub in zip(c[4:], outs):
        assert abs(got - pub) <= 0.5 * 10 ** (math.floor(math.log10(pub)) - 3) + 1e-12
    for got, pub in zip(t[3:], thrs):
        assert abs(got - pub) <= 5e-4
    assert abs(mse - mse_pub) <= 5e-6
    assert resid <= 1e-12


def test_codebook_matches_printed_four_decimals():
    # the four positive centroids as quoted in four decimals: 0.2451, 0.7560, 1.3440, 2.1520
    c, _, _, _ = tq3.lloyd_max_gaussian()
    for got, pub in zip(c[4:], [0.2451, 0.7560, 1.3440, 2.1520]):
        assert abs(got - pub) <= 1e-4


def test_codebook_symmetric_and_fixed_point(cb):
    c, c16, t = cb
    assert np.array_equal(c, -c[::-1])
    assert t[3] == 0.0
    assert np.all(np.diff(c) > 0) and np.all(np.diff(t) > 0)
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-15)
    # c16 are the nearest half-precision values of c
    assert np.all(np.abs(c16 - c) <= np.abs(np.spacing(np.float16(c)).astype(np.float64)) / 2 + 1e-18)


def test_quantizer_mse_closed_form_vs_monte_carlo(cb):
    c, _, t = cb
    z = np.random.default_rng(0).standard_normal(2_000_000)
    q = c[np.searchsorted(t, z, side="right")]
    err = (z - q) ** 2
    mc = err.mean()
    se = err.std() / math.sqrt(len(z))
    assert abs(mc - tq3.quantizer_mse(c, t)) <= 5 * se


# ---- rotation ------------------------------------------------------------------------


@pytest.mark.parametrize("d", [64, 128, 256])
def test_sylvester_hadamard_is_scipy_hadamard(d):
    h = tq3.sylvester_hadamard(d)
    assert np.array_equal(h, scipy.linalg.hadamard(d).astype(np.float64))
    assert np.array_equal(h @ h.T, d * np.eye(d))


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_orthogonal(d):
    signs, _ = splitmix.codec_draws(d, 99)
    pi = tq3.rotation(signs)
    assert np.allclose(pi @ pi.T, np.eye(d), rtol=0, atol=1e-12)
    x = np.random.default_rng(1).standard_normal(d)
    assert abs(np.linalg.norm(pi @ x) - np.linalg.norm(x)) <= 1e-12
    # first basis vector: column 0 of H times D_0 over sqrt(d)
    e = np.zeros(d)
    e[0] = 1.0
    assert np.allclose(pi @ e, signs[0] / math.sqrt(d) * np.ones(d), rtol=0, atol=1e-15)


# ---- encode / decode -------------------------------------------------------------------


@pytest.fixture(scope="module")
def codec128():
    signs, s = splitmix.codec_draws(128, 0x5EED)
    pi = tq3.rotation(signs)
    c, c16, t = tq3.codebook()
    return signs, s, pi, c, c16, t


def test_threshold_rule_is_nearest_centroid(codec128):
    _, s, pi, c, c16, t = codec128
    rng = np.random.default_rng(2)
    for _ in range(50):
        x = rng.standard_normal(128) * rng.uniform(0.1, 10)
        rec = tq3.encode(x, True, pi, s, c16, t)
        brute = np.argmin(np.abs(rec["z"][:, None] - c[None, :]), axis=1)
        assert np.array_equal(rec["code"], brute)


def test_ties_go_up(codec128):
    _, _, _, _, _, t = codec128
    for j, tj in enumerate(t):
        assert int(np.sum(t <= tj)) == j + 1


def test_zero_vector(codec128):
    _, s, pi, _, c16, t = codec128
    rec = tq3.encode(np.zeros(128), True, pi, s, c16, t)
    assert np.all(rec["code"] == 4)
    assert rec["n16"] == 0.0 and rec["g16"] == 0.0
    assert np.all(rec["bits"] == 1)


def test_bit_budget_matches_page(golden):
    rows = dict((r[0], float(r[1])) for r in golden("tq3_bit_budget.txt"))
    assert tq3.record_bytes(128, True) * 8 / 128 == rows["key_bits_per_dim"]
    assert tq3.record_bytes(128, False) * 8 / 128 == rows["value_bits_per_dim"]
    overall = (tq3.record_bytes(128, True) + tq3.record_bytes(128, False)) * 8 / 256
    assert abs(overall - rows["overall_approx"]) < 0.1
    assert tq3.record_bytes(128, True) == 68 and tq3.record_bytes(128, False) == 50


def test_fp16_saturating_rounding():
    assert tq3.fp16_sat(1.0 + 2.0 ** -11) == 1.0  # tie goes to even
    assert tq3.fp16_sat(1.0 + 3 * 2.0 ** -11) == 1.0 + 2.0 ** -9
    assert tq3.fp16_sat(65519.0) == 65504.0
    assert tq3.fp16_sat(65520.0) == 65504.0  # would round to inf: saturates
    assert tq3.fp16_sat(1e9) == 65504.0
    assert tq3.fp16_sat(2.0 ** -24) == 2.0 ** -24


def test_value_reconstruction_error(codec128):
    # E|x - v_hat|^2 / |x|^2 is the quantizer's MSE per coordinate over d
    # coordinates of variance 1/d each: about 0.0345 (plus tiny fp16 effects).
    _, s, pi, c, c16, t = codec128
    rng = np.random.default_rng(3)
    errs = []
    for _ in range(400):
        x = rng.standard_normal(128)
        rec = tq3.encode(x, False, pi, s, c16, t)
        vh = tq3.decode_value(rec["code"], rec["n16"], pi, c16)
        errs.append(np.sum((x - vh) ** 2) / np.sum(x * x))
    assert abs(np.mean(errs) - tq3.quantizer_mse(c, t)) < 0.003


def test_key_decode_factored_form(codec128):
    # <q, k_eff> equals the kernel's factored score n16/sqrt(d) <Pi q, c16[code]>
    # + g16 sqrt(pi/2)/d <S Pi q, b>.
    _, s, pi, _, c16, t = codec128
    rng = np.random.default_rng(4)
    for _ in range(20):
        x, q = rng.standard_normal(128), rng.standard_normal(128)
        rec = tq3.encode(x, True, pi, s, c16, t)
        k_eff = tq3.decode_key(rec["code"], rec["bits"], rec["n16"], rec["g16"], pi, s, c16)
        q1 = pi @ q
        q2 = s.astype(np.float64) @ q1
        b = np.where(rec["bits"] != 0, 1.0, -1.0)
        fact = rec["n16"] / math.sqrt(128) * (q1 @ c16[rec["code"]]) + rec["g16"] * math.sqrt(math.pi / 2) / 128 * (q2 @ b)
        assert abs(q @ k_eff - fact) <= 1e-11


def test_qjl_estimate_unbiased(codec128):
    # With q, x and D fixed and S drawn afresh T times, the mean of <q, k_eff>
    # equals <q, x> (the QJL identity E[sign(<s,r>) <s,y>] = sqrt(2/pi) <r,y>/|r|),
    # up to the fp16 rounding of |r|, within 5 standard errors.
    signs, _, pi, _, c16, t = codec128
    rng = np.random.default_rng(5)
    x, q = rng.standard_normal(128), rng.standard_normal(128)
    vals, qjl = [], []
    T = 6000
    for _ in range(T):
        s_mat = rng.standard_normal((128, 128)).astype(np.float32)
        rec = tq3.encode(x, True, pi, s_mat, c16, t)
        k_eff = tq3.decode_key(rec["code"], rec["bits"], rec["n16"], rec["g16"], pi, s_mat, c16)
        k_mse = tq3.decode_value(rec["code"], rec["n16"], pi, c16)
        vals.append(q @ k_eff)
        qjl.append(q @ (k_eff - k_mse))
    vals, qjl = np.array(vals), np.array(qjl)
    se = vals.std() / math.sqrt(T)
    assert abs(vals.mean() - q @ x) <= 5 * se + 0.01
    # the same draws without the sqrt(pi/2) factor are clearly biased
    biased = vals - qjl * (1.0 - math.sqrt(2.0 / math.pi))
    assert abs(biased.mean() - q @ x) > 5 * se + 0.01


# ---- SplitMix64 and the seeded draws ----------------------------------------------------


def test_splitmix64_reference_outputs(golden):
    g = splitmix.SplitMix64(0)
    for row in golden("splitmix64_seed0.txt"):
        assert g.next() == int(row[0], 16)


def test_free_list_order():
    assert splitmix.free_list_order(10, 0) == list(range(10))
    perm = splitmix.free_list_order(1000, 77)
    assert sorted(perm) == list(range(1000)) and perm != list(range(1000))
    assert splitmix.free_list_order(1000, 77) == perm


def test_codec_draw_statistics():
    signs, s = splitmix.codec_draws(128, 0x5EED)
    assert set(np.unique(signs)) <= {-1, 1}
    assert abs(int(signs.sum())) <= 5 * math.sqrt(128)
    flat = s.astype(np.float64).ravel()
    n = flat.size
    assert abs(flat.mean()) <= 5 / math.sqrt(n)
    assert abs(flat.var() - 1.0) <= 5 * math.sqrt(2.0 / n)
    # Gaussian fourth moment 3
    assert abs(np.mean(flat ** 4) - 3.0) <= 5 * math.sqrt(96.0 / n)


def test_batch_encode_decode_match_per_vector(codec128):
    _, s, pi, _, c16, t = codec128
    rng = np.random.default_rng(9)
    xs = rng.standard_normal((64, 128)) * rng.uniform(0.2, 5, size=(64, 1))
    xs[3] = 0.0
    for is_key in (True, False):
        batch = tq3.encode_batch(xs, is_key, pi, s, c16, t, chunk=17)
        for i, x in enumerate(xs):
            one = tq3.encode(x, is_key, pi, s, c16, t)
            assert np.array_equal(batch["code"][i], one["code"])
            assert batch["n16"][i] == one["n16"]
            if is_key:
                assert np.array_equal(batch["bits"][i], one["bits"])
                assert batch["g16"][i] == one["g16"]
                kb = tq3.decode_keys(batch["code"][i:i + 1], batch["bits"][i:i + 1], batch["n16"][i:i + 1],
                                     batch["g16"][i:i + 1], pi, s, c16)[0]
                ko = tq3.decode_key(one["code"], one["bits"], one["n16"], one["g16"], pi, s, c16)
                assert np.allclose(kb, ko, rtol=0, atol=1e-12)
            else:
                vb = tq3.decode_values(batch["code"][i:i + 1], batch["n16"][i:i + 1], pi, c16)[0]
                assert np.allclose(vb, tq3.decode_value(one["code"], one["n16"], pi, c16), rtol=0, atol=1e-12)
