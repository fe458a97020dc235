"""Verify-step attention of one sequence, written as its definition, in fp64.

What the pages fix:
* AX Engine page, "Core Technical Architecture & Methods": up to 4 draft tokens
  per step are checked by one forward pass of the target model, so a verify
  step carries 1 + k <= 5 query rows per sequence.  The SwiftLM page's
  speculative-decoding passage says the same: the main model checks N+1
  positions at once.
* AX Engine page, "Supported Model Families": Qwen3-4B uses dense grouped-query
  attention; Gemma4 uses sliding-window plus full attention layers and a soft
  cap on the logits.
* mlx-engine blog, section on current model architectures: Gemma 4's local
  layers use a 512-token sliding window, interleaved with global layers.

Readings (the pages never write the formula):
* plain scaled-dot-product softmax attention per query head; the scale is a
  parameter (1/sqrt(d) in every workload here).
* the k draft rows are appended before verification, so row i of a sequence
  whose cache now holds L positions sits at position p_i = L - n + i, and sees
  keys j <= p_i (itself and earlier drafts included).
* query head h reads kv head h // g with g = Hq / Hkv (contiguous groups).
* window W > 0: key j is visible from p iff 0 <= p - j < W (W keys, self
  included); W = 0 means no window.
* soft cap c > 0 is applied to the scaled score, before masking:
  s <- c * tanh(s / c); c = 0 means no cap.
"""

import numpy as np


def visible_keys(p, window):
    """Indices j of the keys position p can see."""
    lo = 0 if window == 0 else max(0, p - window + 1)
    return np.arange(lo, p + 1)


def verify_attention(q, k, v, scale, softcap=0.0, window=0, return_weights=False):
    """Attention of the n = q.shape[0] newest positions of one sequence.

    q: [n, Hq, d]; k, v: [L, Hkv, d] (L >= n, the full cache after the append).
    Returns o: [n, Hq, d] in fp64 (and, if asked, a dict (i, h) -> (keys,
    weights)).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    assert L >= n and hq % hkv == 0
    g = hq // hkv
    out = np.zeros((n, hq, d), dtype=np.float64)
    weights = {}
    for i in range(n):
        p = L - n + i
        keys = visible_keys(p, window)  # a contiguous range lo..p
        lo, hi = int(keys[0]), int(keys[-1]) + 1
        for h in range(hq):
            kv = h // g
            s = scale * (k[lo:hi, kv, :] @ q[i, h, :])
            if softcap > 0.0:
                s = softcap * np.tanh(s / softcap)
            e = np.exp(s - s.max())
            w = e / e.sum()
            out[i, h, :] = w @ v[lo:hi, kv, :]
            if return_weights:
                weights[(i, h)] = (keys, w)
    if return_weights:
        return out, weights
    return out


def verify_attention_grouped(q, k, v, scale, softcap=0.0, window=0, return_weights=False):
    """The same attention as ``verify_attention``, arranged per kv head: the
    scores of all n rows and g query heads of kv head h against every key
    some row can see form one matrix (a single matrix product), each row's
    invisible keys are masked out explicitly, and each column goes through
    its own max-subtracted softmax.  Nothing is blocked, fused or reordered
    beyond that grouping, so each entry is the definition's value; it is
    here because long sequences are too slow row by row.
    """
    q = np.asarray(q, dtype=np.float64)
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    assert L >= n and hq % hkv == 0
    g = hq // hkv
    first = L - n
    lo = 0 if window == 0 else max(0, first - window + 1)
    keys = np.arange(lo, L)
    pos = first + np.arange(n)
    vis = keys[None, :] <= pos[:, None]
    if window > 0:
        vis &= (pos[:, None] - keys[None, :]) < window
    vis = np.repeat(vis, g, axis=0)  # row i * g + j: row i, query head h * g + j
    out = np.zeros((n, hq, d), dtype=np.float64)
    weights = {}
    for h in range(hkv):
        qh = q[:, h * g:(h + 1) * g, :].reshape(n * g, d)
        # fp64 copies of one kv head at a time (the caller's arrays may be fp32)
        kh = np.asarray(k[lo:, h, :], dtype=np.float64)
        vh = np.asarray(v[lo:, h, :], dtype=np.float64)
        s = scale * (qh @ kh.T)
        if softcap > 0.0:
            s = softcap * np.tanh(s / softcap)
        s = np.where(vis, s, -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        w = e / e.sum(axis=1, keepdims=True)
        out[:, h * g:(h + 1) * g, :] = (w @ vh).reshape(n, g, d)
        if return_weights:
            for r in range(n * g):
                i, j = divmod(r, g)
                weights[(i, h * g + j)] = (keys[vis[r]], w[r, vis[r]])
    if return_weights:
        return out, weights
    return out


def verify_attention_batch(qs, ks, vs, scale, softcap=0.0, window=0):
    """One call over several sequences: lists of per-sequence arrays."""
    return [verify_attention(q, k, v, scale, softcap, window) for q, k, v in zip(qs, ks, vs)]


def visible_key_count(L, n, window):
    """Number of distinct keys some row of the sequence can see (the union of
    the rows' visible sets): the bytes a reader of the cache must fetch."""
    first = L - n
    lo = 0 if window == 0 else max(0, first - window + 1)
    return L - lo
