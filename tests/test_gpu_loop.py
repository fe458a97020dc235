"""One speculative decode loop through every piece, on the GPU: the n-gram
drafter proposes drafts (host), kv_append_verify appends and verifies the
1 + k rows, spec_accept (greedy) decides against target logits, and
kv_rollback_device drops the rejected rows without the host.

The target "model" is a known token stream per sequence (periodic with
substitutions): row j of a sequence that has committed P tokens scores the
stream's token P + 1 + j highest.  So the accepted counts, the next tokens
and the final lengths have exact host expectations; the attention outputs
of every step are checked for finiteness here and against the oracle in the
other GPU tests.
"""

import numpy as np
import pytest
import torch

from parity import require_gpu
from speculative_verify_attention_amd import KV_BF16, KVCache, NgramDrafter, accept, synth

pytestmark = pytest.mark.gpu

VOCAB = 512


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def streams(n_seqs, length, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n_seqs):
        period = rng.integers(0, VOCAB, size=rng.integers(5, 10))
        s = np.resize(period, length)
        noise = rng.random(length) < 0.08
        s[noise] = rng.integers(0, VOCAB, size=noise.sum())
        out.append(s.tolist())
    return out


def test_decode_loop_with_ngram_drafts_and_device_rollback():
    print("[case] decode loop: drafter -> append_verify -> accept -> device rollback", flush=True)
    prefill = [300, 40, 1000, 255]
    n = len(prefill)
    wl = synth.Workload("loop", 8, 2, 128, KV_BF16, prefill, [5] * n, seed=77, steps=40)
    cache = KVCache(wl.hkv, wl.d, wl.num_blocks(), n, wl.max_blocks_per_seq(), KV_BF16)
    for s, L in enumerate(prefill):
        k, v = synth.prefill_kv(wl, s, 0, L, "cuda")
        cache.append([s], [L], k, v)
    truth = streams(n, 2000, 5)
    drafter = NgramDrafter(n, max_drafts=4)
    committed = list(prefill)  # tokens in the cache; token `committed` is the last output, not yet cached
    for s in range(n):
        drafter.observe(s, truth[s][: committed[s] + 1])
    seqs = list(range(n))
    accepted_total = drafted_total = 0
    for step in range(30):
        drafts = drafter.draft_batch(seqs)
        rows = [1 + len(d) for d in drafts]
        k, v = synth.step_kv(wl, step, sum(rows), "cuda")
        q = synth.queries(wl, step, sum(rows), "cuda")
        out = cache.append_verify(seqs, rows, k, v, q, wl.hq, wl.scale)
        # target logits: row j of sequence s prefers the stream's token committed + 1 + j
        target = torch.randn((sum(rows), VOCAB), device="cuda")
        r0 = 0
        for s in seqs:
            for j in range(rows[s]):
                target[r0 + j, truth[s][committed[s] + 1 + j]] += 20.0
            r0 += rows[s]
        draft_tok = torch.tensor([t for d in drafts for t in d] or [0], dtype=torch.int32, device="cuda")
        u = torch.zeros(sum(rows), device="cuda")
        acc, tok = accept([len(d) for d in drafts], target, draft_tok, u, 0.0)
        cache.rollback_device(seqs, [len(d) for d in drafts], acc)
        acc_h, tok_h = acc.cpu().tolist(), tok.cpu().tolist()  # the drafter is host code
        assert torch.isfinite(out).all()
        for s in seqs:
            want = 0
            while want < len(drafts[s]) and drafts[s][want] == truth[s][committed[s] + 1 + want]:
                want += 1
            assert acc_h[s] == want, (step, s)
            assert tok_h[s] == truth[s][committed[s] + 1 + want], (step, s)
            drafter.observe(s, drafts[s][:want] + [tok_h[s]])
            committed[s] += 1 + want
            accepted_total += want
            drafted_total += len(drafts[s])
    cache.sync()
    assert [cache.seq_len(s) for s in seqs] == committed
    rate = accepted_total / max(1, drafted_total)
    print(f"accepted {accepted_total} of {drafted_total} drafts ({rate:.2f})", flush=True)
    assert rate > 0.5  # periodic streams with 8% substitutions are mostly predictable
