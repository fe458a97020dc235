"""The compressed KV-cache codec ("TQ3"), encode and decode, in fp64.

What the pages fix (SwiftLM page, TurboQuant KV-cache compression passage):
* the cache is compressed online, at about 3.6 bits per coordinate;
* keys take 3-bit codes plus a 1-bit QJL residual: 4.25 bits per dimension;
* values take 3-bit codes only: 3.125 bits per dimension; values get no QJL
  because they never enter the inner-product scores;
* the 3-bit codes come from a nonlinear Lloyd-Max codebook, encoded natively
  and dequantized inside the attention kernel.

The exact format is not on the pages.  The reading taken here, for a vector
x in R^d (d a power of two):
* rotation Pi = H_d * diag(D) / sqrt(d): H_d the Sylvester Hadamard matrix,
  D the seeded +-1 signs (``splitmix.codec_draws``);
* n = ||x||, y = Pi (x / n), z = sqrt(d) * y, so the coordinates of z are close
  to N(0, 1);
* code_i = number of Lloyd-Max decision thresholds t_j with t_j <= z_i (ties go
  up), in 0..7;
* the stored reconstruction levels are the 8-level Gaussian Lloyd-Max
  centroids rounded to IEEE half precision, c16 = fp16(c): exactly the values
  the attention kernel multiplies;
* n16 = fp16(n), round to nearest even, saturating at 65504;
* keys only: r = Pi x - n16 * c16[code] / sqrt(d) (the residual against what the
  decoder rebuilds), gamma16 = fp16(||r||), bit_i = [(S r)_i >= 0] with S the
  seeded d x d Gaussian matrix;
* decode: value v_hat = Pi^T (n16 * c16[code] / sqrt(d)); key
  k_eff = Pi^T (n16 * c16[code] / sqrt(d) + gamma16 * sqrt(pi/2) / d * S^T b),
  b_i = +1 if bit_i else -1.  With S Gaussian, E[sign(<s, r>) <s, y>] =
  sqrt(2/pi) <r, y> / ||r||, so <q, k_eff> is an unbiased estimate of
  <q, Pi^T (n16 c16/sqrt(d) + r)> (the QJL estimator with m = d projections).
* storage per vector: key d/2 bytes (code + sign bit per dimension) + two fp16
  scalars; value 3d/8 bytes + one fp16 scalar.  At d = 128 that is 68 B and
  50 B: 4.25 and 3.125 bits per dimension, the page's budgets.
"""

import math

import numpy as np
from scipy.special import ndtr

FP16_MAX = 65504.0


# --- Lloyd-Max codebook ---------------------------------------------------------


def _phi(x):
    return np.where(np.isinf(x), 0.0, np.exp(-0.5 * np.where(np.isinf(x), 0.0, x) ** 2) / math.sqrt(2.0 * math.pi))


def lloyd_max_gaussian(levels=8, tol=1e-15, max_iter=200000):
    """Lloyd-Max quantizer for N(0, 1): alternate the two optimality
    conditions (each threshold is the midpoint of its neighbouring levels;
    each level is the conditional mean of its cell) until the levels stop
    moving.  Returns (levels c, thresholds t, mean-squared error, fixed-point
    residual)."""
    c = np.linspace(-2.0, 2.0, levels)
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        a = np.concatenate(([-np.inf], t))
        b = np.concatenate((t, [np.inf]))
        mass = ndtr(b) - ndtr(a)
        c_new = (_phi(a) - _phi(b)) / mass
        c_new = 0.5 * (c_new - c_new[::-1])  # N(0,1) is symmetric: keep c odd
        step = np.max(np.abs(c_new - c))
        c = c_new
        if step < tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    a = np.concatenate(([-np.inf], t))
    b = np.concatenate((t, [np.inf]))
    mass = ndtr(b) - ndtr(a)
    resid = np.max(np.abs((_phi(a) - _phi(b)) / mass - c))
    return c, t, quantizer_mse(c, t), resid


def quantizer_mse(c, t):
    """E[(Z - c[q(Z)])^2] for Z ~ N(0,1), from the closed-form moments of a
    truncated normal on each cell [a, b]:
      int z^2 phi = Phi(b) - Phi(a) - (b phi(b) - a phi(a)),
      int z phi = phi(a) - phi(b)."""
    a = np.concatenate(([-np.inf], t))
    b = np.concatenate((t, [np.inf]))
    mass = ndtr(b) - ndtr(a)
    aphi = np.where(np.isinf(a), 0.0, np.where(np.isinf(a), 0.0, a) * _phi(a))
    bphi = np.where(np.isinf(b), 0.0, np.where(np.isinf(b), 0.0, b) * _phi(b))
    m2 = mass - (bphi - aphi)
    m1 = _phi(a) - _phi(b)
    return float(np.sum(m2 - 2.0 * c * m1 + c * c * mass))


def codebook():
    """(c exact fp64, c16 stored levels as fp64 values of fp16, thresholds)."""
    c, t, _, _ = lloyd_max_gaussian()
    c16 = c.astype(np.float16).astype(np.float64)
    return c, c16, t


# --- rotation -------------------------------------------------------------------


def sylvester_hadamard(d):
    """H_1 = [1]; H_2m = [[H_m, H_m], [H_m, -H_m]] (Kronecker products)."""
    assert d > 0 and d & (d - 1) == 0
    h = np.array([[1.0]])
    base = np.array([[1.0, 1.0], [1.0, -1.0]])
    while h.shape[0] < d:
        h = np.kron(base, h)
    return h


def rotation(signs):
    """Pi = H_d diag(D) / sqrt(d)."""
    d = len(signs)
    return sylvester_hadamard(d) @ np.diag(np.asarray(signs, dtype=np.float64)) / math.sqrt(d)


# --- scalar fp16 ----------------------------------------------------------------


def fp16_sat(x):
    """Round a non-negative fp64 to half precision (nearest, ties to even),
    saturating at the largest finite half."""
    with np.errstate(over="ignore"):
        h = np.float16(x)
    if np.isinf(h):
        return FP16_MAX
    return float(h)


# --- encode / decode ------------------------------------------------------------


def encode(x, is_key, pi, s_mat, c16, t):
    """Encode one vector.  Returns dict(code[d] uint8, n16, and for keys
    bits[d] uint8 and g16)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[0]
    n = math.sqrt(float(np.sum(x * x)))
    y = np.zeros(d) if n == 0.0 else pi @ (x / n)
    z = math.sqrt(d) * y
    code = np.array([int(np.sum(t <= zi)) for zi in z], dtype=np.uint8)
    n16 = fp16_sat(n)
    rec = {"code": code, "n16": n16, "z": z, "n": n}
    if is_key:
        r = pi @ x - n16 * c16[code] / math.sqrt(d)
        rho = math.sqrt(float(np.sum(r * r)))
        proj = s_mat.astype(np.float64) @ r
        rec["bits"] = (proj >= 0.0).astype(np.uint8)
        rec["g16"] = fp16_sat(rho)
        rec["proj"] = proj
        rec["rho"] = rho
    return rec


def decode_value(code, n16, pi, c16):
    d = len(code)
    return pi.T @ (n16 * c16[np.asarray(code)] / math.sqrt(d))


def decode_key(code, bits, n16, g16, pi, s_mat, c16):
    d = len(code)
    b = np.where(np.asarray(bits) != 0, 1.0, -1.0)
    mse_part = n16 * c16[np.asarray(code)] / math.sqrt(d)
    qjl_part = g16 * math.sqrt(math.pi / 2.0) / d * (s_mat.astype(np.float64).T @ b)
    return pi.T @ (mse_part + qjl_part)


def encode_many(xs, is_key, pi, s_mat, c16, t):
    return [encode(x, is_key, pi, s_mat, c16, t) for x in xs]


def record_bytes(d, is_key):
    """Stored bytes per vector: keys carry a 3-bit code and a sign bit per
    dimension plus two fp16 scalars; values a 3-bit code per dimension plus
    one fp16 scalar."""
    if is_key:
        return (4 * d) // 8 + 2 + 2
    return (3 * d) // 8 + 2


# --- the same steps over many vectors at once --------------------------------------
#
# encode_batch / decode_batch apply exactly the per-vector steps above to the
# rows of a matrix (each row independent; the matrix products are the
# per-vector products stacked).  tests/test_oracle_tq3.py pins them to the
# per-vector functions.


def fp16_sat_array(x):
    with np.errstate(over="ignore"):
        h = np.asarray(x, dtype=np.float64).astype(np.float16)
    h = np.where(np.isinf(h), np.float16(FP16_MAX), h)
    return h.astype(np.float64)


def encode_batch(xs, is_key, pi, s_mat, c16, t, chunk=65536):
    """Encode the rows of xs [N, d]: dict of arrays code [N, d] uint8, n16 [N],
    z [N, d], and for keys bits [N, d] uint8, g16 [N], proj [N, d]."""
    xs = np.asarray(xs, dtype=np.float64)
    N, d = xs.shape
    out = {"code": np.empty((N, d), np.uint8), "n16": np.empty(N), "z": np.empty((N, d)), "n": np.empty(N)}
    if is_key:
        out.update(bits=np.empty((N, d), np.uint8), g16=np.empty(N), proj=np.empty((N, d)), rho=np.empty(N))
    s64 = s_mat.astype(np.float64)
    for a in range(0, N, chunk):
        x = xs[a: a + chunk]
        n = np.sqrt(np.sum(x * x, axis=1))
        safe = np.where(n == 0.0, 1.0, n)
        y = (x / safe[:, None]) @ pi.T
        y[n == 0.0] = 0.0
        z = math.sqrt(d) * y
        code = np.zeros(z.shape, dtype=np.uint8)
        for tj in t:
            code += (tj <= z).astype(np.uint8)
        n16 = fp16_sat_array(n)
        out["code"][a: a + chunk] = code
        out["n16"][a: a + chunk] = n16
        out["z"][a: a + chunk] = z
        out["n"][a: a + chunk] = n
        if is_key:
            r = x @ pi.T - n16[:, None] * c16[code] / math.sqrt(d)
            rho = np.sqrt(np.sum(r * r, axis=1))
            proj = r @ s64.T
            out["bits"][a: a + chunk] = (proj >= 0.0).astype(np.uint8)
            out["g16"][a: a + chunk] = fp16_sat_array(rho)
            out["proj"][a: a + chunk] = proj
            out["rho"][a: a + chunk] = rho
    return out


def decode_values(code, n16, pi, c16):
    """Rows of decoded values: Pi^T (n16 c16[code] / sqrt(d))."""
    d = code.shape[1]
    return (n16[:, None] * c16[code] / math.sqrt(d)) @ pi


def decode_keys(code, bits, n16, g16, pi, s_mat, c16):
    """Rows of decoded keys: Pi^T (n16 c16[code]/sqrt(d) + g16 sqrt(pi/2)/d S^T b)."""
    d = code.shape[1]
    b = np.where(bits != 0, 1.0, -1.0)
    rot = n16[:, None] * c16[code] / math.sqrt(d) + g16[:, None] * math.sqrt(math.pi / 2.0) / d * (b @ s_mat.astype(np.float64))
    return rot @ pi
