"""Helpers for the GPU parity tests: oracle expectations for a Runner's state
and readback of the cache's stored bytes through the documented pool layout."""

import math

import numpy as np

from oracle import attention as A


def require_gpu():
    import pytest
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU: the HIP path cannot be exercised here")


def qoffsets(rows):
    off = [0]
    for n in rows:
        off.append(off[-1] + n)
    return off


def oracle_seq(runner, s, rows, q_host, layer):
    """fp64 oracle output [rows[s], hq, d] of sequence s."""
    wl = runner.wl
    window, cap = runner.layers[layer]
    off = qoffsets(rows)
    k, v = runner.logical_kv(s)
    return A.verify_attention(q_host[off[s]: off[s + 1]], k, v, wl.scale, cap, window)


def max_err(runner, rows, q, out, layer, seqs):
    """Max |gpu - oracle| over the given sequences (all rows, all heads)."""
    q_host = q.float().cpu().numpy().astype(np.float64)
    o_host = out.float().cpu().numpy().astype(np.float64)
    off = qoffsets(rows)
    worst = 0.0
    for s in seqs:
        ref = oracle_seq(runner, s, rows, q_host, layer)
        got = o_host[off[s]: off[s + 1]]
        assert np.all(np.isfinite(got)), f"non-finite output for sequence {s}"
        worst = max(worst, float(np.max(np.abs(got - ref))))
    return worst


def read_plain(cache, s, L):
    """K, V [L, hkv, d] of sequence s read from an fp32/bf16 pool via the
    documented layout (K [hkv][256][d]; V [hkv][4][d][64] per block)."""
    import torch

    hkv, d = cache.num_kv_heads, cache.head_dim
    dt = torch.float32 if cache.fmt == 0 else torch.bfloat16
    e = 4 if cache.fmt == 0 else 2
    half = hkv * 256 * d * e
    bb = 2 * half
    table = cache.block_table(s)
    ks, vs = [], []
    for b in range(math.ceil(L / 256)):
        base = table[b] * bb
        kb = cache.pool[base: base + half].view(dt).reshape(hkv, 256, d).permute(1, 0, 2)
        vb = cache.pool[base + half: base + bb].view(dt).reshape(hkv, 4, d, 64).permute(1, 3, 0, 2)
        ks.append(kb)
        vs.append(vb.reshape(256, hkv, d))
    return torch.cat(ks)[:L], torch.cat(vs)[:L]
