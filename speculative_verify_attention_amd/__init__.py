"""Speculative-verify attention over a paged, rollback-able KV cache, for
MI355X (gfx950).

The work runs in ``libsvattn.so`` (C ABI in ``include/svattn.h``): a
deterministic host block manager with 256-token blocks and O(1) rollback,
slice-update and quantize-on-append kernels, and a split-context MFMA
attention kernel with its log-sum-exp merge, and the acceptance step that
follows it (greedy or rejection sampling).  This package is the Python
binding (argument marshalling only) plus the seeded synthetic-input
generators in ``synth``.
"""

from ._binding import (  # noqa: F401
    KV_BF16,
    KV_BLOCK_SIZE,
    KV_EDEVICE,
    KV_EINVAL,
    KV_ENOMEM,
    KV_ENOSEQ,
    KV_ERANGE,
    KV_FP32,
    KV_MAX_ROWS,
    KV_OK,
    KV_TQ3,
    KVCache,
    NgramDrafter,
    SvattnError,
    accept,
    core_lib,
    ngram_params,
    kv_append,
    kv_block_table,
    kv_codec,
    kv_create,
    kv_destroy,
    kv_encode,
    kv_free_blocks,
    kv_last_error,
    kv_params,
    kv_pool_bytes,
    kv_record_bytes,
    kv_rollback,
    kv_rollback_batch,
    kv_trace_events,
    kv_seq_free,
    kv_seq_len,
    kv_workspace_bytes,
    kv_workspace_bytes_valu,
    lib,
    spec_accept,
    spec_accept_workspace_bytes,
    spec_verify_attn,
    spec_verify_attn_valu,
    svcore_params,
)
