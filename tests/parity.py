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


def unswizzle_subtiles(raw, fmt, D, kind):
    """Undo the documented sub-tile order of a plain-format K or V region:
    raw [n_sub, 32 * D] -> [n_sub * 32 tokens, D]."""
    n = raw.shape[0]
    if fmt == 1 and kind == "k":  # (kk, h, m, e) = K[m][16kk + 8h + e]
        t = raw.reshape(n, D // 16, 2, 32, 8).permute(0, 3, 1, 2, 4)
    elif fmt == 1:  # (v, dt, h, r, e1, e0) = V[16v + 8e1 + 4h + e0][32dt + r]
        t = raw.reshape(n, 2, D // 32, 2, 32, 2, 4).permute(0, 1, 5, 3, 6, 2, 4)
    elif kind == "k":  # (kq, h, m, e) = K[m][(D/2)h + 4kq + e]
        t = raw.reshape(n, D // 8, 2, 32, 4).permute(0, 3, 2, 1, 4)
    else:  # (uq, dt, h, r, e) = V[8uq + 4h + e][32dt + r]
        t = raw.reshape(n, 4, D // 32, 2, 32, 4).permute(0, 1, 3, 5, 2, 4)
    return t.reshape(n * 32, D)


def read_plain(cache, s, L):
    """K, V [L, hkv, d] of sequence s read from an fp32/bf16 pool through the
    documented layout (per block: every head's K region, then every head's V
    region; each region is 8 sub-tiles of 32 tokens in MFMA operand order)."""
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
        kb = cache.pool[base: base + half].view(dt).reshape(hkv, 8, 32 * d)
        vb = cache.pool[base + half: base + bb].view(dt).reshape(hkv, 8, 32 * d)
        ks.append(torch.stack([unswizzle_subtiles(kb[h], cache.fmt, d, "k") for h in range(hkv)], dim=1))
        vs.append(torch.stack([unswizzle_subtiles(vb[h], cache.fmt, d, "v") for h in range(hkv)], dim=1))
    return torch.cat(ks)[:L], torch.cat(vs)[:L]
