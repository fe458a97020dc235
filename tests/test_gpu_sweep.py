"""Seeded sweep of random configurations through the C ABI: format (fp32,
bf16, TQ3), head dim, GQA group, number of sequences, context lengths
(log-uniform in 8..3000), rows drawn per step (1..5), rollbacks (0..4) before
each step, window and soft cap; odd cases append and verify in one call
(kv_append_verify).  Three steps per configuration; every
output of the last step is checked against the fp64 oracle at the usual
bars (1e-5 fp32 and TQ3, 2e-3 bf16).  Many small random cases reach value-
and shape-dependent corners (exact fp16 ties, ragged tails, chunk splits)
that the named cases do not."""

import numpy as np
import pytest
import torch

from parity import max_err, max_err_tq3, require_gpu
from speculative_verify_attention_amd import KV_BF16, KV_FP32, KV_TQ3, synth
from speculative_verify_attention_amd.runner import Runner

pytestmark = pytest.mark.gpu

TOL = {KV_FP32: 1e-5, KV_BF16: 2e-3, KV_TQ3: 1e-5}
N_CASES = 96


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def config(i):
    rng = np.random.default_rng(1000 + i)
    fmt = (KV_FP32, KV_BF16, KV_TQ3)[i % 3]
    d = int(rng.choice([64, 128] if fmt == KV_TQ3 else [64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))  # rows <= 5: at most 40 query columns per kv head
    n = int(rng.integers(1, 13))
    # at least 8 positions, so that a rollback of up to 4 never exceeds a length
    prefill = np.exp(rng.uniform(np.log(8.0), np.log(3000.0), n)).astype(int).tolist()
    window = int(rng.choice([0, 0, int(rng.integers(1, 1200))]))
    cap = float(rng.choice([0.0, 0.0, 30.0]))
    return synth.Workload(f"sweep{i}", hkv * g, hkv, d, fmt, prefill, [1] * n, window=window, softcap=cap, seed=i,
                          alloc_seed=i + 1, codec_seed=0x5EED, steps=3, vary_rows=True, rollback_max=4)


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep(i):
    wl = config(i)
    print(f"[case] sweep {i} ({'fused' if i % 2 else 'separate'}): fmt={wl.fmt} d={wl.d} hq={wl.hq} hkv={wl.hkv} seqs={wl.n_seqs} "
          f"window={wl.window} cap={wl.softcap} prefill={wl.prefill}", flush=True)
    r = Runner(wl, track=True)
    r.fill()
    for t in range(wl.steps):
        rows, q, outs = r.step(t, fused=(i % 2 == 1))
    torch.cuda.synchronize()
    f = max_err_tq3 if wl.fmt == KV_TQ3 else max_err
    err = f(r, rows, q, outs[0], 0, range(wl.n_seqs))
    print(f"max abs err {err:.3e}", flush=True)
    assert err <= TOL[wl.fmt], err
