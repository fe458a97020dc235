"""Acceptance of draft tokens after a verify forward, in fp64.

Test infrastructure only (see the package header).  Written from the
SwiftLM page, speculative-decoding passage: drafts are checked against the
target model with probabilistic rejection sampling as Leviathan et al.
define it -- the ratio P_target / P_draft decides each draft and a rejected
position is re-sampled from the corrected distribution -- so that the output
follows the target distribution at non-zero temperature; and, as the same
page says of another decoder, greedy decoding takes the argmax and ignores
the temperature.  The AX Engine page ("Core Technical Architecture &
Methods") drafts with n-gram tables, which give no draft distribution: such
a draft is a point mass on its token.

Readings taken (the pages fix none of them):
* sequence s verifies n drafts d_0..d_{n-1}; target row j (j = 0..n) is the
  target's distribution for the j-th token after the last accepted one, so
  row j checks draft j and row n gives the bonus token;
* temperature T > 0: p = softmax(logits / T), the draft's q likewise; T = 0:
  greedy -- accept d_j while it equals the first index of the maximum of row
  j; the first mismatch outputs that argmax, and if every draft passes, the
  argmax of row n follows;
* sampling: draft j is accepted iff u_j * q_j(d_j) < p_j(d_j) (the test
  u < p / q without a division); the first rejection stops the run and
  draws from r(x) = max(0, p_j(x) - q_j(x)); if every draft passes, the draw
  is from p_n; the draw uses u_n;
* a draw from an unnormalized weight vector w with uniform u returns the
  smallest token t with sum_{x <= t} w(x) > u * sum_x w(x) (tokens in index
  order).
"""

import numpy as np


def softmax_t(logits, temperature):
    """softmax(logits / T) in fp64, max-subtracted."""
    x = np.asarray(logits, dtype=np.float64) / float(temperature)
    x = x - x.max()
    e = np.exp(x)
    return e / e.sum()


def first_argmax(row):
    """Index of the first maximum (ties go to the lowest index)."""
    row = np.asarray(row)
    return int(np.flatnonzero(row == row.max())[0])


def draw(weights, u):
    """Smallest t with cumsum(w)[t] > u * sum(w); weights >= 0, sum > 0."""
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    idx = np.flatnonzero(c > u * c[-1])
    return int(idx[0]) if idx.size else int(np.flatnonzero(w > 0)[-1])


def accept_one(target, draft_logits, drafts, uniforms, temperature):
    """One sequence.  target: [n+1, V] logits; draft_logits: [n, V] or None
    (point-mass drafts); drafts: [n] tokens; uniforms: [n+1] in [0, 1).
    Returns (accepted, token, info) where info records, for the parity test,
    the margins of every decision taken."""
    target = np.asarray(target, dtype=np.float64)
    n = len(drafts)
    info = {"ratio_margin": [], "draw": None}
    if temperature == 0.0:
        for j in range(n):
            a = first_argmax(target[j])
            if drafts[j] != a:
                return j, a, info
        return n, first_argmax(target[n]), info
    for j in range(n):
        p = softmax_t(target[j], temperature)
        q = softmax_t(draft_logits[j], temperature) if draft_logits is not None else None
        d = int(drafts[j])
        qd = q[d] if q is not None else 1.0
        info["ratio_margin"].append((uniforms[j] * qd - p[d]) / max(p[d], 1e-300))
        if not uniforms[j] * qd < p[d]:
            if q is not None:
                r = np.maximum(0.0, p - q)
            else:
                r = p.copy()
                r[d] = 0.0
            info["draw"] = (r, uniforms[n])
            return j, draw(r, uniforms[n]), info
    p = softmax_t(target[n], temperature)
    info["draw"] = (p, uniforms[n])
    return n, draw(p, uniforms[n]), info


def accept_batch(target_rows, draft_rows, drafts, uniforms, n_draft, temperature):
    """All sequences: target_rows [sum(n+1), V], draft_rows [sum(n), V] or
    None, drafts [sum(n)], uniforms [sum(n+1)].  Returns (accepted, tokens,
    infos) lists in sequence order."""
    acc, tok, infos = [], [], []
    t0 = d0 = 0
    for n in n_draft:
        a, t, info = accept_one(target_rows[t0:t0 + n + 1],
                                None if draft_rows is None else draft_rows[d0:d0 + n],
                                drafts[d0:d0 + n], uniforms[t0:t0 + n + 1], temperature)
        acc.append(a)
        tok.append(t)
        infos.append(info)
        t0 += n + 1
        d0 += n
    return acc, tok, infos
