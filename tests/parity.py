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
    return A.verify_attention_grouped(q_host[off[s]: off[s + 1]], k, v, wl.scale, cap, window)


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


# ---- compressed (TQ3) cache ------------------------------------------------------------


def oracle_codec(d, codec_seed):
    """The oracle's own codec: (pi, S, c, c16, t, signs), drawn from the seed."""
    from oracle import splitmix, tq3

    signs, s_mat = splitmix.codec_draws(d, codec_seed)
    c, c16, t = tq3.codebook()
    return tq3.rotation(signs), s_mat, c, c16, t, signs


def _tq3_maps(d):
    nb = 16 * d
    j, h, m, kq, b = np.unravel_index(np.arange(nb), (d // 64, 2, 32, 4, 4))
    k_m = m
    k_dim = 16 * (4 * j + kq) + 8 * h + 2 * b
    planes = d // 64
    pj, ph, pr, half = np.unravel_index(np.arange(planes * 2 * 32 * 2), (planes, 2, 32, 2))
    v_off = 16 * d + pj * 768 + (32 * ph + pr) * 12 + half * 6
    v_dim = 32 * (2 * pj + half) + pr
    q = np.arange(16)
    v_tok = 16 * (q[None, :] >> 3) + 8 * ((q[None, :] & 7) >> 2) + 4 * ph[:, None] + (q[None, :] & 3)
    i = np.arange(16)
    s_tok = np.stack([8 * (i >> 2) + 4 * hh + (i & 3) for hh in (0, 1)])  # [h, i]
    return k_m, k_dim, v_off, v_dim, v_tok, s_tok


def read_tq3(cache, s, L):
    """Logical TQ3 fields of sequence s, positions [0, L), read from the pool
    through the documented layout: dict of arrays kcode, kbit [L, hkv, d],
    kn16, kg16 [L, hkv], vcode [L, hkv, d], vn16 [L, hkv]."""
    hkv, d = cache.num_kv_heads, cache.head_dim
    sb = 28 * d + 192
    bb = hkv * 8 * sb
    table = cache.block_table(s)
    nblk = math.ceil(L / 256)
    pool = cache.pool
    raw = np.stack([pool[table[b] * bb: table[b] * bb + bb].cpu().numpy() for b in range(nblk)])  # [nblk, bb]
    raw = raw.reshape(nblk, hkv, 8, sb).transpose(0, 2, 3, 1)  # [blk, sub, byte, head]
    raw = raw.reshape(nblk * 8, sb, hkv)  # [sub-tile, byte, head]
    nsub = raw.shape[0]
    k_m, k_dim, v_off, v_dim, v_tok, s_tok = _tq3_maps(d)
    kcode = np.zeros((nsub, 32, hkv, d), np.uint8)
    kbit = np.zeros_like(kcode)
    kb = raw[:, : 16 * d, :]  # [sub, byte, head]
    lo, hi = kb & 15, kb >> 4
    kcode[:, k_m, :, k_dim] = (lo & 7).transpose(1, 0, 2)
    kbit[:, k_m, :, k_dim] = (lo >> 3).transpose(1, 0, 2)
    kcode[:, k_m, :, k_dim + 1] = (hi & 7).transpose(1, 0, 2)
    kbit[:, k_m, :, k_dim + 1] = (hi >> 3).transpose(1, 0, 2)
    vcode = np.zeros((nsub, 32, hkv, d), np.uint8)
    fields = np.zeros((nsub, len(v_off), hkv), np.uint64)
    for b in range(6):
        fields |= raw[:, v_off + b, :].astype(np.uint64) << np.uint64(8 * b)
    for qi in range(16):
        codes = ((fields >> np.uint64(3 * qi)) & np.uint64(7)).astype(np.uint8)  # [sub, field, head]
        vcode[:, v_tok[:, qi], :, v_dim] = codes.transpose(1, 0, 2)
    sc = raw[:, 28 * d: 28 * d + 192, :].copy()
    sc16 = sc.reshape(nsub, 2, 3, 16, 2, hkv)
    vals = (sc16[..., 0, :].astype(np.uint16) | (sc16[..., 1, :].astype(np.uint16) << 8)).view(np.float16)
    kn16 = np.zeros((nsub, 32, hkv))
    kg16 = np.zeros_like(kn16)
    vn16 = np.zeros_like(kn16)
    for hh in (0, 1):
        kn16[:, s_tok[hh], :] = vals[:, hh, 0].astype(np.float64)
        kg16[:, s_tok[hh], :] = vals[:, hh, 1].astype(np.float64)
        vn16[:, s_tok[hh], :] = vals[:, hh, 2].astype(np.float64)
    flat = lambda x: x.reshape((nsub * 32,) + x.shape[2:])[:L]  # noqa: E731
    return {"kcode": flat(kcode), "kbit": flat(kbit), "kn16": flat(kn16), "kg16": flat(kg16),
            "vcode": flat(vcode), "vn16": flat(vn16)}


def half_ulp(x):
    with np.errstate(over="ignore"):  # values past the fp16 range have an infinite spacing
        return np.spacing(np.asarray(x, dtype=np.float64).astype(np.float16)).astype(np.float64)


def compare_tq3_fields(gpu, ora, is_key, band=1e-5):
    """Bit-exact comparison of encoded fields with the decision-boundary
    exclusions: codes whose z lies within `band` of a threshold, sign bits
    whose projection lies within `band` of 0, norms within band*ulp16 of a
    rounding midpoint; a vector with an excluded code has its sign bits and
    residual norm excluded too.  Returns (mismatches, excluded, total)."""
    from oracle import tq3

    _, _, t = tq3.codebook()
    z = ora["z"]
    near_t = np.min(np.abs(z[..., None] - t), axis=-1) < band
    code_ok = (gpu["code"] == ora["code"]) | near_t
    mism = int(np.sum(~code_ok))
    excl = int(np.sum(near_t & (gpu["code"] != ora["code"])))
    total = z.size
    n = ora["n"]
    mid = np.abs(n - ora["n16"]) - half_ulp(ora["n16"]) / 2
    n_ok = (gpu["n16"] == ora["n16"]) | (np.abs(mid) < band * half_ulp(ora["n16"]))
    mism += int(np.sum(~n_ok))
    if is_key:
        vec_excl = np.any(near_t, axis=-1)
        proj = ora["proj"]
        near0 = (np.abs(proj) < band) | vec_excl[..., None]
        bit_ok = (gpu["bits"] == ora["bits"]) | near0
        mism += int(np.sum(~bit_ok))
        excl += int(np.sum(near0 & (gpu["bits"] != ora["bits"])))
        rho = ora["rho"]
        gmid = np.abs(rho - ora["g16"]) - half_ulp(ora["g16"]) / 2
        g_ok = (gpu["g16"] == ora["g16"]) | (np.abs(gmid) < band * half_ulp(ora["g16"])) | vec_excl
        mism += int(np.sum(~g_ok))
    return mism, excl, total


def unpack_records(rec, d, is_key):
    """kv_encode records [N, bytes] (uint8 numpy) -> dict of logical fields."""
    N = rec.shape[0]
    if is_key:
        nib = np.empty((N, d), np.uint8)
        nib[:, 0::2] = rec[:, : d // 2] & 15
        nib[:, 1::2] = rec[:, : d // 2] >> 4
        n16 = (rec[:, d // 2].astype(np.uint16) | (rec[:, d // 2 + 1].astype(np.uint16) << 8)).view(np.float16)
        g16 = (rec[:, d // 2 + 2].astype(np.uint16) | (rec[:, d // 2 + 3].astype(np.uint16) << 8)).view(np.float16)
        return {"code": nib & 7, "bits": nib >> 3, "n16": n16.astype(np.float64), "g16": g16.astype(np.float64)}
    nbytes = 3 * d // 8
    bits = np.unpackbits(rec[:, :nbytes], axis=1, bitorder="little")  # [N, 3d]
    code = (bits[:, 0::3] | (bits[:, 1::3] << 1) | (bits[:, 2::3] << 2)).astype(np.uint8)
    n16 = (rec[:, nbytes].astype(np.uint16) | (rec[:, nbytes + 1].astype(np.uint16) << 8)).view(np.float16)
    return {"code": code, "n16": n16.astype(np.float64)}


def tq3_oracle_seq(runner, s, rows, q_host, layer):
    """Oracle output of sequence s of a TQ3 runner: the oracle encodes the same
    fp32 source rows itself, decodes them, and runs its attention."""
    from oracle import tq3

    wl = runner.wl
    window, cap = runner.layers[layer]
    pi, s_mat, _, c16, t, _ = oracle_codec(wl.d, wl.codec_seed)
    k, v = runner.logical_kv(s)
    L = k.shape[0]
    ke = tq3.encode_batch(k.reshape(-1, wl.d), True, pi, s_mat, c16, t)
    ve = tq3.encode_batch(v.reshape(-1, wl.d), False, pi, s_mat, c16, t)
    kd = tq3.decode_keys(ke["code"], ke["bits"], ke["n16"], ke["g16"], pi, s_mat, c16).reshape(L, wl.hkv, wl.d)
    vd = tq3.decode_values(ve["code"], ve["n16"], pi, c16).reshape(L, wl.hkv, wl.d)
    off = qoffsets(rows)
    return A.verify_attention_grouped(q_host[off[s]: off[s + 1]], kd, vd, wl.scale, cap, window)


def max_err_tq3(runner, rows, q, out, layer, seqs):
    q_host = q.float().cpu().numpy().astype(np.float64)
    o_host = out.float().cpu().numpy().astype(np.float64)
    off = qoffsets(rows)
    worst = 0.0
    for s in seqs:
        ref = tq3_oracle_seq(runner, s, rows, q_host, layer)
        got = o_host[off[s]: off[s + 1]]
        assert np.all(np.isfinite(got)), f"non-finite output for sequence {s}"
        worst = max(worst, float(np.max(np.abs(got - ref))))
    return worst
