"""Why the kernels carry queries and probabilities as two parts: an
emulation, in numpy, of the roundings the matrix-core operands apply, against
the same scores and weights in fp64.  For the compressed cache (scores in the
factored form over the stored fp16 levels, signs and norms) the 1e-5 bar
needs q', q'' and P each as fp16 hi + lo; with any one of them as a single
fp16 part a peaked softmax misses it.  For bf16 caches the 2e-3 bar needs the
fp32 queries as two bf16 parts.  Only rounding is emulated: the products are
exact and sums are fp64, as the kernels' fp32 accumulation is far below
these errors.

SwiftLM page, TurboQuant KV-cache compression passage (3-bit codes plus QJL
signs for keys, 3-bit codes for values, dequantized in the attention
kernel); the tolerances are the ones the parity tests use."""

import math

import numpy as np
import pytest
import torch

from oracle import splitmix, tq3

D = 128
TQ3_TOL = 1e-5
BF16_TOL = 2e-3


def f16(x):
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def parts(x, n, rnd):
    """x carried as n parts, each the rounding of what the previous left."""
    out, rest = [], np.asarray(x, np.float64)
    for _ in range(n):
        h = rnd(rest)
        out.append(h)
        rest = rest - h
    return out


@pytest.fixture(scope="module")
def tq3_case():
    """One sequence of 20000 keys, 5 rows x 4 heads of one kv head, queries
    N(0, 4^2): a peaked softmax."""
    rng = np.random.default_rng(11)
    signs, s_mat = splitmix.codec_draws(D, 0x5EED)
    _, c16, t = tq3.codebook()
    pi = tq3.rotation(signs)
    s64 = s_mat.astype(np.float64)
    L, n_rows, g = 20000, 5, 4
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    q = rng.standard_normal((n_rows * g, D)) * 4.0
    ke = tq3.encode_batch(k, True, pi, s_mat, c16, t)
    ve = tq3.encode_batch(v, False, pi, s_mat, c16, t)
    q1 = q @ pi.T
    q2 = (q1 @ s64.T) * math.sqrt(math.pi / 2.0) / math.sqrt(D)
    return dict(a=c16[ke["code"]], b=np.where(ke["bits"] != 0, 1.0, -1.0), n=ke["n16"], gam=ke["g16"],
                cv=c16[ve["code"]], nv=ve["n16"], q1=q1, q2=q2, pi=pi,
                rowpos=np.repeat(np.arange(n_rows), g) + L - n_rows, L=L)


def tq3_out(c, n_q1, n_q2, n_p):
    """Output (rotated back) with q', q'' and P*n_v carried as 1 or 2 fp16 parts."""
    s1 = sum(c["a"] @ p.T for p in parts(c["q1"], n_q1, f16))
    s2 = sum(c["b"] @ p.T for p in parts(c["q2"], n_q2, f16))
    x = (s1 * c["n"][:, None] + s2 * c["gam"][:, None]) / D  # scale 1/sqrt(d), code levels / sqrt(d)
    mask = np.arange(c["L"])[:, None] <= c["rowpos"][None, :]
    x = np.where(mask, x, -np.inf)
    p = np.exp(x - x.max(0))
    w = (p * c["nv"][:, None]).T
    o = sum(pp @ c["cv"] for pp in parts(w, n_p, f16))
    return (o / p.sum(0)[:, None]) / math.sqrt(D) @ c["pi"]


def test_tq3_two_parts_meet_the_bar(tq3_case):
    exact = tq3_out(tq3_case, 3, 3, 3)  # three parts: ~2^-33, the reference
    assert np.max(np.abs(tq3_out(tq3_case, 2, 2, 2) - exact)) <= TQ3_TOL / 2


@pytest.mark.parametrize("one", ["q'", "q''", "P"])
def test_tq3_any_single_part_misses_the_bar(tq3_case, one):
    exact = tq3_out(tq3_case, 3, 3, 3)
    n = {"q'": (1, 2, 2), "q''": (2, 1, 2), "P": (2, 2, 1)}[one]
    assert np.max(np.abs(tq3_out(tq3_case, *n) - exact)) > 4 * TQ3_TOL


def bf16_out(k, v, q, rowpos, n_q, n_p):
    s = sum(p @ k.T for p in parts(q, n_q, bf16)) / math.sqrt(D)
    mask = np.arange(k.shape[0])[None, :] <= rowpos[:, None]
    s = np.where(mask, s, -np.inf)
    p = np.exp(s - s.max(1, keepdims=True))
    o = sum(pp @ v for pp in parts(p, n_p, bf16))
    return o / p.sum(1, keepdims=True)


def test_bf16_queries_need_two_parts():
    """bf16 K/V scaled by 2 (the dense workload's largest head scale), fp32
    queries N(0, 2^2), 3000 keys."""
    rng = np.random.default_rng(12)
    L = 3000
    k = bf16(rng.standard_normal((L, D)) * 2.0)
    v = bf16(rng.standard_normal((L, D)) * 2.0)
    q = rng.standard_normal((20, D)).astype(np.float32).astype(np.float64) * 2.0
    rowpos = np.repeat(np.arange(5), 4) + L - 5
    exact = bf16_out(k, v, q, rowpos, 4, 4)
    assert np.max(np.abs(bf16_out(k, v, q, rowpos, 2, 2) - exact)) <= BF16_TOL / 4
    assert np.max(np.abs(bf16_out(k, v, q, rowpos, 1, 2) - exact)) > 2 * BF16_TOL
