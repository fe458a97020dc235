"""Seeded synthetic inputs for the verify-attention workloads.

This module only draws numbers: it holds none of the method's arithmetic and
is shared by the tests, the benchmark and the oracle checks so that both sides
see the same inputs.  Values are generated with torch generators, chunk by
chunk, so any slice of a long sequence can be regenerated on its own:

* prefill K/V of sequence s, positions [256c, 256c+256): seeded by
  (workload seed, "prefill", s, c);
* the K/V of the rows appended at decode step t: seeded by (seed, "step", t);
* the queries of step t: seeded by (seed, "query", t).

Distributions follow each workload's recipe (N(0,1), optional per-kv-head
scales), and K/V are rounded to the cache's storage type (bf16 caches get
bf16 K/V); queries are plain fp32 draws for every format.

The pages measure end to end on real models (AX Engine page, "Performance
Evidence & Results"; SwiftLM page, long-context benchmark and test-suite
passages at 512 / 40K / 100K tokens, 20 generated tokens per run); no model,
prompt or dataset is used here: these seeded caches of the same shapes stand
in for them.
"""

import dataclasses
import math

import numpy as np

KV_FP32, KV_BF16, KV_TQ3 = 0, 1, 2
BLOCK = 256

_TAG = {"prefill": 1, "step": 2, "query": 3, "scale": 4, "plan": 5, "accept": 6}


def _mix(*parts):
    """Combine integers into one 63-bit generator seed (SplitMix-style
    finaliser; a seed derivation, not part of any computed result)."""
    h = 0x243F6A8885A308D3
    for p in parts:
        h = (h ^ (int(p) & 0xFFFFFFFFFFFFFFFF)) * 0x9E3779B97F4A7C15 & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 31
    return h & 0x7FFFFFFFFFFFFFFF


@dataclasses.dataclass
class Workload:
    name: str
    hq: int
    hkv: int
    d: int
    fmt: int
    prefill: list  # context length of each sequence before the first step
    rows: list  # query rows per sequence at step 0 (1 + drafts)
    window: int = 0
    softcap: float = 0.0
    seed: int = 0
    head_scales: bool = False  # K and V scaled per kv head by U(0.5, 2)
    alloc_seed: int = 0
    codec_seed: int = 0
    steps: int = 1
    vary_rows: bool = False  # rows drawn per step in 1..5 (continuous batching)
    rollback_max: int = 0  # rollback drawn per step in 0..rollback_max before appending

    @property
    def g(self):
        return self.hq // self.hkv

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    @property
    def n_seqs(self):
        return len(self.prefill)

    def torch_dtype(self):
        import torch

        return torch.bfloat16 if self.fmt == KV_BF16 else torch.float32

    def max_blocks_per_seq(self):
        return (max(self.prefill) + 8 * (self.steps + 1) + BLOCK - 1) // BLOCK + 1

    def num_blocks(self):
        return sum((p + 8 * (self.steps + 1) + BLOCK - 1) // BLOCK + 1 for p in self.prefill)


# ---- the workloads ----------------------------------------------------------------------


def tiny():
    """1 sequence, Hq=8, Hkv=2, d=64, fp32 N(0,1), context 256, 5 rows."""
    return Workload("tiny", 8, 2, 64, KV_FP32, [256], [5], seed=1)


def qwen3_4b_dense(batch=16, ctx=4096, seed=2):
    """Qwen3-4B-shaped dense GQA: Hq=32, Hkv=8, d=128, bf16 N(0,1) with a
    per-kv-head scale U(0.5, 2) (drawn separately for K and V)."""
    return Workload("qwen3_4b_dense", 32, 8, 128, KV_BF16, [ctx] * batch, [5] * batch, seed=seed,
                    head_scales=True)


def gemma_interleaved(batch=8, ctx=32768, window=512, seed=3, fmt=KV_BF16):
    """Gemma-style layer: Hq=8, Hkv=1, d=256, soft cap 50; window=512 for the
    local layer, 0 for the global layer; bf16 cache (or the compressed one
    from an fp32 N(0,1) source with fmt=KV_TQ3)."""
    name = ("gemma_window" if window else "gemma_full") + ("_tq3" if fmt == KV_TQ3 else "")
    return Workload(name, 8, 1, 256, fmt, [ctx] * batch, [5] * batch, window=window, softcap=50.0, seed=seed,
                    codec_seed=0x5EED if fmt == KV_TQ3 else 0)


def tq3_long(ctx, batch=4, seed=None, fmt=KV_TQ3):
    """Long context: Hq=32, Hkv=8, d=128, fp32 N(0,1) source, compressed
    (or bf16 with fmt=KV_BF16)."""
    idx = {512: 0, 40000: 1, 100000: 2}.get(ctx, 3)
    return Workload(f"{'tq3' if fmt == KV_TQ3 else 'bf16'}_{ctx}", 32, 8, 128, fmt, [ctx] * batch, [5] * batch,
                    seed=40 + idx if seed is None else seed, codec_seed=0x5EED)


def mixed_batch(n_seqs=64, lo=512, hi=100000, steps=20, seed=5):
    """Continuous-batched mix: lengths log-uniform in [lo, hi], rows uniform
    in 1..5 per sequence per step, rollbacks 0..4 before each step, bf16,
    shuffled block table."""
    rng = np.random.default_rng(_mix(seed, _TAG["plan"]))
    lens = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n_seqs))).astype(int).tolist()
    rows = rng.integers(1, 6, size=n_seqs).tolist()
    return Workload("mixed_batch", 32, 8, 128, KV_BF16, lens, rows, seed=seed, alloc_seed=0xB10C5,
                    steps=steps, vary_rows=True, rollback_max=4)


# ---- draws ---------------------------------------------------------------------------------


def _gen(device, *parts):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(_mix(*parts))
    return g


def head_scales(wl, device="cpu"):
    """(k_scale, v_scale) per kv head, U(0.5, 2), or ones."""
    import torch

    if not wl.head_scales:
        one = torch.ones(wl.hkv, dtype=torch.float32, device=device)
        return one, one
    g = _gen("cpu", wl.seed, _TAG["scale"])
    ks = 0.5 + 1.5 * torch.rand(wl.hkv, generator=g, dtype=torch.float64)
    vs = 0.5 + 1.5 * torch.rand(wl.hkv, generator=g, dtype=torch.float64)
    return ks.float().to(device), vs.float().to(device)


def _finish_kv(wl, k, v, device):
    ks, vs = head_scales(wl, device)
    k = k * ks[None, :, None]
    v = v * vs[None, :, None]
    dt = wl.torch_dtype()
    return k.to(dt), v.to(dt)


def prefill_kv(wl, s, start, count, device):
    """K, V of positions [start, start+count) of sequence s's prefill:
    tensors [count, hkv, d] in the cache's source dtype (bf16 for bf16
    caches, fp32 otherwise)."""
    import torch

    ks, vs = [], []
    c0, c1 = start // BLOCK, (start + count + BLOCK - 1) // BLOCK
    for c in range(c0, c1):
        g = _gen(device, wl.seed, _TAG["prefill"], s, c)
        k = torch.randn((BLOCK, wl.hkv, wl.d), generator=g, device=device, dtype=torch.float32)
        v = torch.randn((BLOCK, wl.hkv, wl.d), generator=g, device=device, dtype=torch.float32)
        ks.append(k)
        vs.append(v)
    k = torch.cat(ks)[start - c0 * BLOCK: start - c0 * BLOCK + count]
    v = torch.cat(vs)[start - c0 * BLOCK: start - c0 * BLOCK + count]
    return _finish_kv(wl, k, v, device)


def step_plan(wl, step):
    """(rollback per sequence, rows per sequence) of decode step `step`.
    Fixed-shape workloads use their own rows and no rollback; continuous-
    batching workloads draw rows in 1..5 and rollbacks in 0..rollback_max
    per sequence per step (the rollback happens before the step's append)."""
    if not (wl.vary_rows or wl.rollback_max):
        return [0] * wl.n_seqs, list(wl.rows)
    rng = np.random.default_rng(_mix(wl.seed, _TAG["plan"], step + 1))
    rows = rng.integers(1, 6, size=wl.n_seqs).tolist() if wl.vary_rows else list(wl.rows)
    rb = rng.integers(0, wl.rollback_max + 1, size=wl.n_seqs).tolist() if wl.rollback_max else [0] * wl.n_seqs
    return rb, rows


def step_kv(wl, step, n_total, device):
    """K, V of the rows appended at step `step` (all sequences, in order):
    [n_total, hkv, d]."""
    import torch

    g = _gen(device, wl.seed, _TAG["step"], step)
    k = torch.randn((n_total, wl.hkv, wl.d), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((n_total, wl.hkv, wl.d), generator=g, device=device, dtype=torch.float32)
    return _finish_kv(wl, k, v, device)


def queries(wl, step, n_total, device, scale=1.0):
    """Queries of step `step`: [n_total, hq, d] fp32 N(0, scale^2), whatever
    the cache format (the boundary takes fp32 queries)."""
    import torch

    g = _gen(device, wl.seed, _TAG["query"], step)
    return torch.randn((n_total, wl.hq, wl.d), generator=g, device=device, dtype=torch.float32) * scale


# ---- inputs of the acceptance step -------------------------------------------------------


def accept_inputs(n_draft, vocab, seed, device, with_draft=True, spread=3.0, noise=0.5, hit=0.7, boost=0.0):
    """Seeded inputs of spec_accept: target logits N(0, spread^2) per row,
    draft logits = the matching target row + N(0, noise^2) (a draft model
    close to the target) with `boost` added at the drafted token (a draft
    model surer of its token than the target), draft tokens = the target
    row's largest logit with probability `hit`, else a uniform token, and
    uniforms in [0, 1).
    Returns (target [sum(n+1), vocab], draft [sum(n), vocab] or None,
    tokens int32 [sum(n)], uniforms [sum(n+1)])."""
    import torch

    rows_t, rows_d = sum(n_draft) + len(n_draft), sum(n_draft)
    g = _gen(device, seed, _TAG["accept"])
    target = torch.randn((rows_t, vocab), generator=g, device=device, dtype=torch.float32) * spread
    # the target row that checks each draft
    check = []
    t0 = 0
    for n in n_draft:
        check.extend(range(t0, t0 + n))
        t0 += n + 1
    check = torch.tensor(check, dtype=torch.int64, device=device)
    draft = None
    if with_draft:
        draft = target[check] + torch.randn((rows_d, vocab), generator=g, device=device, dtype=torch.float32) * noise
    top = target[check].argmax(dim=1).to(torch.int32) if rows_d else torch.zeros(0, dtype=torch.int32, device=device)
    rnd = torch.randint(0, vocab, (rows_d,), generator=g, device=device, dtype=torch.int32)
    keep = torch.rand((rows_d,), generator=g, device=device) < hit
    tokens = torch.where(keep, top, rnd).contiguous()
    if draft is not None and boost and rows_d:
        draft[torch.arange(rows_d, device=device), tokens.long()] += boost
    uniforms = torch.rand((rows_t,), generator=g, device=device, dtype=torch.float32)
    return target.contiguous(), draft, tokens, uniforms
