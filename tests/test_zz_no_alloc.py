"""spec_verify_attn_static (the verify call on the library's fixed device
scratch, which allocates nothing) against spec_verify_attn with a workspace
of the caller's: the same kernels on the same inputs, so the outputs must be
equal bit for bit.  Two calls in a row on each cache, the second smaller than
the first (fewer sequences, fewer rows), so the second runs over scratch the
first left behind.  A call that needs more scratch than the fixed array holds
is refused before anything is launched."""

import pytest
import torch

from parity import require_gpu
from speculative_verify_attention_amd import KV_BF16, KV_ENOMEM, KVCache, SvattnError, synth
from speculative_verify_attention_amd.runner import Runner

pytestmark = pytest.mark.gpu

STATIC_BYTES = 32 << 20


def banner(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def both(cache, wl, seqs, rows, q, window, cap):
    need = cache.workspace_bytes(seqs, rows, wl.hq, window)
    assert need <= STATIC_BYTES, need
    ref = cache.verify(seqs, rows, q, wl.hq, wl.scale, cap, window)
    got = cache.verify_static(seqs, rows, q, wl.hq, wl.scale, cap, window)
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), float((got - ref).abs().max())


CASES = [
    ("tq3 4x8192", lambda: synth.tq3_long(8192, batch=4), None),
    ("qwen3-4b bf16 8x4096", lambda: synth.qwen3_4b_dense(batch=8, ctx=4096), None),
    ("gemma window 512 cap 50, 4x8192", lambda: synth.gemma_interleaved(batch=4, ctx=8192, window=512), None),
    ("mixed batch 24 seqs", lambda: synth.mixed_batch(n_seqs=24, lo=256, hi=30000, steps=1), None),
]


@pytest.mark.parametrize("name,make,_", CASES, ids=[c[0] for c in CASES])
def test_static_matches_workspace_two_calls(name, make, _):
    wl = make()
    banner(f"no-alloc verify: {name}")
    r = Runner(wl)
    r.fill()
    rb, rows = r.plan(0)
    r.rollback(rb)
    r.append_rows(0, rows)
    cache = r.caches[0]
    window, cap = r.layers[0]
    seqs = list(range(wl.n_seqs))
    q = r.queries(0, rows)
    both(cache, wl, seqs, rows, q, window, cap)
    # second call: every other sequence, in reverse order, one or two rows each
    seqs2 = seqs[::-2]
    rows2 = [1 + (i % 2) for i in range(len(seqs2))]
    q2 = synth.queries(wl, 1, sum(rows2), "cuda")
    both(cache, wl, seqs2, rows2, q2, window, cap)


def test_static_refuses_oversize_call():
    banner("no-alloc verify: oversize call refused")
    hkv, d, n = 8, 128, 256
    c = KVCache(hkv, d, n, n, 1, KV_BF16)
    k = torch.randn(8 * n, hkv, d, device="cuda").to(torch.bfloat16)
    c.append(list(range(n)), [8] * n, k, k)
    seqs, rows = list(range(n)), [8] * n
    hq = 64  # 8 rows x 8 query heads per kv head: 64 rows per tile
    assert c.workspace_bytes(seqs, rows, hq) > STATIC_BYTES
    q = torch.randn(8 * n, hq, d, device="cuda")
    with pytest.raises(SvattnError) as ei:
        c.verify_static(seqs, rows, q, hq, d ** -0.5)
    assert ei.value.code == KV_ENOMEM
    # the refusal leaves the cache usable: a call that fits still matches
    few, frows = seqs[:16], [8] * 16
    assert c.workspace_bytes(few, frows, hq) <= STATIC_BYTES
    ref = c.verify(few, frows, q[:128].contiguous(), hq, d ** -0.5)
    got = c.verify_static(few, frows, q[:128].contiguous(), hq, d ** -0.5)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
