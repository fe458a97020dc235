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


# Pins of the seeded draws.  Each takes the function under test, so that the
# planted mistakes below can be run through the same pins.

GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def _pin_fisher_yates_scripted(fy):
    # hand-worked Fisher-Yates over [0, 5) with scripted draws 7, 7, 7, 7:
    # i=4: 7 mod 5 = 2, swap 4,2 -> 0 1 4 3 2; i=3: 7 mod 4 = 3, stays;
    # i=2: 7 mod 3 = 1, swap 2,1 -> 0 4 1 3 2; i=1: 7 mod 2 = 1, stays
    it = iter([7, 7, 7, 7])
    assert fy(5, lambda: next(it)) == [0, 4, 1, 3, 2]
    # draws 1, 2, 3, 4: i=4: 1 mod 5 = 1 -> 0 4 2 3 1; i=3: 2 mod 4 = 2 ->
    # 0 4 3 2 1; i=2: 3 mod 3 = 0 -> 3 4 0 2 1; i=1: 4 mod 2 = 0 -> 4 3 0 2 1
    it = iter([1, 2, 3, 4])
    assert fy(5, lambda: next(it)) == [4, 3, 0, 2, 1]


def _pin_free_list_golden(fy):
    # seeded with the golden gamma, SplitMix64's state after its first step is
    # that of seed 0 after one output, so the shuffle draws the golden outputs
    # 2..4 of seed 0: j = 0x...65f4 mod 4 = 0 (last hex digit 4), then
    # 0x06c45d188009454f mod 3 = 1 (16 = 1 mod 3, hex digit sum 94), then
    # 0x...81ec mod 2 = 0: 0 1 2 3 -> 3 1 2 0 -> 3 2 1 0 -> 2 3 1 0
    assert fy(4, splitmix.SplitMix64(GOLDEN_GAMMA).next) == [2, 3, 1, 0]


def _pin_box_muller_closed_forms(bm):
    top = (1 << 64) - 1
    # u1 = 1 exactly (the +1 keeps u1 in (0, 1]): rho = 0
    assert bm(top, 0) == (0.0, 0.0)
    # u1 = 2^-53, u2 = 0: (sqrt(-2 ln 2^-53), 0) = (sqrt(106 ln 2), 0)
    a, b = bm(0, 0)
    assert abs(a - math.sqrt(106.0 * math.log(2.0))) <= 1e-12 and b == 0.0
    # u1 = 1/2 (x1 >> 11 = 2^52 - 1), u2 = 1/4: a quarter turn, (0, sqrt(2 ln 2))
    r = math.sqrt(2.0 * math.log(2.0))
    a, b = bm((1 << 63) - (1 << 11), 1 << 62)
    assert abs(a) <= 1e-15 and abs(b - r) <= 1e-15
    # u2 = 1/2: a half turn, (-sqrt(2 ln 2), 0)
    a, b = bm((1 << 63) - (1 << 11), 1 << 63)
    assert abs(a + r) <= 1e-15 and abs(b) <= 1e-15


def _pin_codec_draws_scripted(cd):
    # d = 2: two sign outputs (top bit set and clear, low bits the other way
    # round), then the pairs of S in row-major order: (u1 = 1/2, u2 = 1/4) for
    # row 0, (u1 = 1, u2 = 0) for row 1
    top = (1 << 64) - 1
    it = iter([1 << 63, 1, (1 << 63) - (1 << 11), 1 << 62, top, 0])
    signs, s = cd(2, lambda: next(it))
    assert signs.tolist() == [-1, 1]
    assert abs(float(s[0, 0])) <= 1e-15
    assert s[0, 1] == np.float32(math.sqrt(2.0 * math.log(2.0)))
    assert s[1, 0] == 0.0 and s[1, 1] == 0.0


def _pin_codec_signs_golden(cd):
    # the top bits of the golden outputs of seed 0: 0xe2.., 0x6e.., 0x06.., 0xf8..
    signs, _ = cd(4, splitmix.SplitMix64(0).next)
    assert signs.tolist() == [-1, 1, 1, -1]


def test_free_list_order():
    assert splitmix.free_list_order(10, 0) == list(range(10))
    perm = splitmix.free_list_order(1000, 77)
    assert sorted(perm) == list(range(1000)) and perm != list(range(1000))
    assert splitmix.free_list_order(1000, 77) == perm
    _pin_fisher_yates_scripted(splitmix.fisher_yates)
    _pin_free_list_golden(splitmix.fisher_yates)
    assert splitmix.free_list_order(4, GOLDEN_GAMMA) == [2, 3, 1, 0]


def test_codec_draws_pins():
    _pin_box_muller_closed_forms(splitmix.box_muller)
    _pin_codec_draws_scripted(splitmix.codec_draws_stream)
    _pin_codec_signs_golden(splitmix.codec_draws_stream)
    signs, s = splitmix.codec_draws(4, 0)
    assert signs.tolist() == [-1, 1, 1, -1]
    # the first pair of S comes from the 5th and 6th outputs, row-major
    g = splitmix.SplitMix64(0)
    outs = [g.next() for _ in range(6)]
    a, b = splitmix.box_muller(outs[4], outs[5])
    assert s[0, 0] == np.float32(a) and s[0, 1] == np.float32(b)


def _fy_mutant(kind):
    def fy(n, draw):
        order = list(range(n))
        steps = range(1, n) if kind == "upward" else range(n - 1, 0, -1)
        for i in steps:
            j = draw() % (i if kind == "mod_i" else i + 1)
            order[i], order[j] = order[j], order[i]
        return order

    return fy


def _bm_mutant(kind):
    def bm(x1, x2):
        u1 = ((x1 >> 11) + (0 if kind == "no_plus_one" else 1)) * 2.0 ** -53
        u2 = (x2 >> 11) * 2.0 ** -53
        rho = math.sqrt(-2.0 * math.log(u1)) if u1 > 0 else math.inf
        c, sn = math.cos(2.0 * math.pi * u2), math.sin(2.0 * math.pi * u2)
        return (rho * sn, rho * c) if kind == "cos_sin_swapped" else (rho * c, rho * sn)

    return bm


def _cd_mutant(kind):
    bm = _bm_mutant(kind)

    def cd(d, draw):
        signs = np.empty(d, dtype=np.int8)
        for i in range(d):
            x = draw()
            signs[i] = -1 if ((x & 1) if kind == "low_bit_sign" else (x >> 63)) else 1
        flat = np.empty(d * d, dtype=np.float32)
        for t in range(0, d * d, 2):
            x1, x2 = draw(), draw()
            with np.errstate(all="ignore"):
                a, b = bm(x1, x2)
                flat[t], flat[t + 1] = np.float32(a), np.float32(b)
        s = flat.reshape(d, d)
        return signs, (s.T.copy() if kind == "column_major" else s)

    return cd


@pytest.mark.parametrize("kind", ["mod_i", "upward"])
def test_free_list_pins_catch_planted_mistake(kind):
    bad = _fy_mutant(kind)
    caught = []
    for pin in (_pin_fisher_yates_scripted, _pin_free_list_golden):
        try:
            pin(bad)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the '{kind}' mistake"


@pytest.mark.parametrize("kind", ["low_bit_sign", "cos_sin_swapped", "no_plus_one", "column_major"])
def test_codec_draw_pins_catch_planted_mistake(kind):
    caught = []
    for pin, fn in ((_pin_box_muller_closed_forms, _bm_mutant(kind)), (_pin_codec_draws_scripted, _cd_mutant(kind)),
                    (_pin_codec_signs_golden, _cd_mutant(kind))):
        try:
            pin(fn)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the '{kind}' mistake"


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
