"""Drive a synthetic workload through the C ABI: create the layer caches,
fill them with the prefill, then run decode steps (rollback, append the new
rows, verify).  Orchestration only: every computed value comes from the
library.

With ``track=True`` the runner also records, for every cached position, where
its K/V came from (a prefill position or a row of some step), so that a
checker can rebuild the logical cache contents without reading the device.
"""

import math

import numpy as np

from . import synth
from ._binding import KVCache


def ring_blocks_per_seq(window):
    """Blocks a ring cache with this window keeps per sequence at most: the
    last window + 8 positions, from a block boundary."""
    return ceil_div(window + 8 - 1 + 255, 256)


class Runner:
    def __init__(self, wl, layers=None, device="cuda", track=False, extra_blocks=0, ring=False):
        """layers: list of (window, softcap) per layer handle; default one
        layer with the workload's own window and cap.  ring: window layers
        get ring caches (memory for their last window + 8 positions only)."""
        self.wl = wl
        self.device = device
        self.layers = layers or [(wl.window, wl.softcap)]
        self.caches = []
        for window, _ in self.layers:
            rw = window if (ring and window > 0) else 0
            nb = (wl.n_seqs * ring_blocks_per_seq(rw) if rw else wl.num_blocks()) + extra_blocks
            self.caches.append(KVCache(wl.hkv, wl.d, nb, wl.n_seqs, wl.max_blocks_per_seq(), wl.fmt, wl.alloc_seed,
                                       wl.codec_seed, device=device, ring_window=rw))
        self.track = track
        self.prov = [np.zeros(0, dtype=np.int64) for _ in range(wl.n_seqs)]  # -1-p: prefill p; r >= 0: step row r
        self.step_k, self.step_v = [], []  # host copies of step rows (tracked runs)
        self.step_rows0 = 0

    # -- setup ---------------------------------------------------------------------
    def fill(self, chunk_rows=1 << 16):
        """Append every sequence's prefill, in calls of at most chunk_rows rows."""
        import torch

        wl = self.wl
        for s, L in enumerate(wl.prefill):
            for start in range(0, L, chunk_rows):
                cnt = min(chunk_rows, L - start)
                k, v = synth.prefill_kv(wl, s, start, cnt, self.device)
                for c in self.caches:
                    c.append([s], [cnt], k, v)
            if self.track:
                self.prov[s] = -1 - np.arange(L, dtype=np.int64)
        torch.cuda.synchronize()

    # -- one decode step ----------------------------------------------------------------
    def plan(self, step):
        return synth.step_plan(self.wl, step)

    def rollback(self, rb):
        if not any(rb):
            return
        seqs = [s for s, r in enumerate(rb) if r]
        for c in self.caches:
            c.rollback_batch(seqs, [rb[s] for s in seqs])
        if self.track:
            for s in seqs:
                self.prov[s] = self.prov[s][: len(self.prov[s]) - rb[s]]

    def append_rows(self, step, rows):
        wl = self.wl
        n_total = int(sum(rows))
        k, v = synth.step_kv(wl, step, n_total, self.device)
        seqs = list(range(wl.n_seqs))
        for c in self.caches:
            c.append(seqs, rows, k, v)
        self._record(k, v, rows)
        return k, v

    def _record(self, k, v, rows):
        """Provenance of appended rows (tracked runs)."""
        if self.track:
            self.step_k.append(k.float().cpu().numpy())
            self.step_v.append(v.float().cpu().numpy())
            off = self.step_rows0
            for s, n in enumerate(rows):
                self.prov[s] = np.concatenate([self.prov[s], off + np.arange(n, dtype=np.int64)])
                off += n
            self.step_rows0 = off

    def queries(self, step, rows, scale=1.0):
        return synth.queries(self.wl, step, int(sum(rows)), self.device, scale)

    def verify(self, layer, rows, q, out=None, workspace=None, stream=None):
        window, cap = self.layers[layer]
        c = self.caches[layer]
        return c.verify(list(range(self.wl.n_seqs)), rows, q, self.wl.hq, self.wl.scale, cap, window, out=out,
                        workspace=workspace, stream=stream)

    def step(self, step, scale_q=1.0, fused=False):
        """rollback -> append -> verify on every layer (fused: kv_append_verify);
        returns (rows, q, outs)."""
        rb, rows = self.plan(step)
        self.rollback(rb)
        if not fused:
            self.append_rows(step, rows)
            q = self.queries(step, rows, scale_q)
            outs = [self.verify(i, rows, q) for i in range(len(self.layers))]
            return rows, q, outs
        wl = self.wl
        k, v = synth.step_kv(wl, step, int(sum(rows)), self.device)
        q = self.queries(step, rows, scale_q)
        seqs = list(range(wl.n_seqs))
        outs = [c.append_verify(seqs, rows, k, v, q, wl.hq, wl.scale, cap, window)
                for c, (window, cap) in zip(self.caches, self.layers)]
        self._record(k, v, rows)
        return rows, q, outs

    # -- logical contents (tracked runs) ----------------------------------------------------
    def logical_kv(self, s):
        """Host fp32 K, V [seq_len, hkv, d] of sequence s as the cache should hold
        them, rebuilt from the recorded provenance."""
        prov = self.prov[s]
        L = len(prov)
        pre = -1 - prov[prov < 0]
        k = np.zeros((L, self.wl.hkv, self.wl.d), dtype=np.float32)
        v = np.zeros_like(k)
        if len(pre):
            hi = int(pre.max()) + 1
            pk, pv = synth.prefill_kv(self.wl, s, 0, hi, self.device)
            pk, pv = pk.float().cpu().numpy(), pv.float().cpu().numpy()
            m = prov < 0
            k[m] = pk[pre]
            v[m] = pv[pre]
        if self.step_k:
            allk = np.concatenate(self.step_k)
            allv = np.concatenate(self.step_v)
            m = prov >= 0
            k[m] = allk[prov[m]]
            v[m] = allv[prov[m]]
        return k, v


def alg_bytes_per_call(wl, rows, lens, window):
    """Stored bytes of the keys some row of each sequence can see, summed over
    sequences and kv heads (K and V): the bytes a reader must fetch."""
    per_tok = {0: 8 * wl.d, 1: 4 * wl.d, 2: (wl.d // 2 + 4) + (3 * wl.d // 8 + 2)}[wl.fmt]
    total = 0
    for L, n in zip(lens, rows):
        lo = 0 if window == 0 else max(0, L - n - window + 1)
        total += (L - lo) * wl.hkv * per_tok
    return total


def ceil_div(a, b):
    return -(-a // b)


__all__ = ["Runner", "alg_bytes_per_call", "ceil_div", "math", "ring_blocks_per_seq"]
