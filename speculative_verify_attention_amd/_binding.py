"""ctypes binding of libsvattn.so (include/svattn.h).

Argument marshalling only: every step of the path runs in the library's
kernels.  Functions keep the C names; ``KVCache`` bundles a handle with the
torch tensors that own its device memory (torch is used for allocation and
streams only).  If the library is not built the calls raise; nothing falls
back to another implementation.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, always (no environment override)
LIB_PATH = os.path.join(PKG, "libsvattn.so")
CORE_LIB_PATH = os.path.join(PKG, "libsvattn_core.so")

KV_OK, KV_EINVAL, KV_ENOMEM, KV_ERANGE, KV_ENOSEQ, KV_EDEVICE = 0, -1, -2, -3, -4, -5
KV_FP32, KV_BF16, KV_TQ3 = 0, 1, 2
KV_BLOCK_SIZE = 256
KV_MAX_ROWS = 8
STATUS_NAMES = {0: "KV_OK", -1: "KV_EINVAL", -2: "KV_ENOMEM", -3: "KV_ERANGE", -4: "KV_ENOSEQ", -5: "KV_EDEVICE"}

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)


class kv_params(ctypes.Structure):
    _fields_ = [
        ("num_kv_heads", _i32),
        ("head_dim", _i32),
        ("block_size", _i32),
        ("num_blocks", _i32),
        ("max_seqs", _i32),
        ("max_blocks_per_seq", _i32),
        ("format", _i32),
        ("ring_window", _i32),
        ("alloc_seed", ctypes.c_uint64),
        ("codec_seed", ctypes.c_uint64),
        ("pool", _p),
        ("pool_bytes", ctypes.c_size_t),
    ]


class ngram_params(ctypes.Structure):
    _fields_ = [
        ("max_seqs", _i32),
        ("max_drafts", _i32),
        ("ema_tau", ctypes.c_double),
        ("ema_threshold", ctypes.c_double),
    ]


class svcore_params(ctypes.Structure):
    _fields_ = [
        ("num_kv_heads", _i32),
        ("head_dim", _i32),
        ("block_size", _i32),
        ("num_blocks", _i32),
        ("max_seqs", _i32),
        ("max_blocks_per_seq", _i32),
        ("format", _i32),
        ("ring_window", _i32),
        ("alloc_seed", ctypes.c_uint64),
        ("codec_seed", ctypes.c_uint64),
    ]


class SvattnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


_LIB = None
_CORE = None

_SIGS = {
    "kv_pool_bytes": [ctypes.POINTER(kv_params), ctypes.POINTER(ctypes.c_size_t)],
    "kv_create": [ctypes.POINTER(kv_params), _p, ctypes.POINTER(_p)],
    "kv_destroy": [_p],
    "kv_append": [_p, _i32, _i32p, _i32p, _p, _p, _p],
    "kv_rollback": [_p, _i32, _i32],
    "kv_rollback_batch": [_p, _i32, _i32p, _i32p],
    "kv_trace_events": [_p, _p, _p],
    "kv_seq_free": [_p, _i32],
    "kv_encode": [_p, _i64, _p, _i32, _p, _p],
    "kv_record_bytes": [_i32, _i32, _i32p],
    "kv_workspace_bytes": [_p, _i32, _i32p, _i32p, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)],
    "spec_verify_attn": [_p, _i32, _i32p, _i32p, _p, _i32, ctypes.c_float, ctypes.c_float, _i32, _p, _p,
                         ctypes.c_size_t, _p],
    "kv_workspace_bytes_valu": [_p, _i32, _i32p, _i32p, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)],
    "spec_verify_attn_valu": [_p, _i32, _i32p, _i32p, _p, _i32, ctypes.c_float, ctypes.c_float, _i32, _p, _p,
                              ctypes.c_size_t, _p],
    "kv_append_verify": [_p, _i32, _i32p, _i32p, _p, _p, _p, _i32, ctypes.c_float, ctypes.c_float, _i32, _p, _p,
                         ctypes.c_size_t, _p],
    "kv_append_verify_workspace_bytes": [_p, _i32, _i32p, _i32p, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)],
    "kv_rollback_device": [_p, _i32, _i32p, _i32p, _p, _p],
    "kv_sync": [_p],
    "kv_seq_len": [_p, _i32, _i32p],
    "kv_block_table": [_p, _i32, _i32p, _i32, _i32p],
    "kv_free_blocks": [_p, _i32p],
    "kv_codec": [_p, _p, _p, _p, _p, _p],
    "kv_last_error": [_p],
    "spec_accept": [_i32, _i32p, _i32, _p, _p, _p, _p, ctypes.c_float, _p, _p, _p, ctypes.c_size_t, _p],
    "spec_accept_workspace_bytes": [_i32, _i32p, _i32, _i32, ctypes.c_float, ctypes.POINTER(ctypes.c_size_t)],
    "spec_accept_last_error": [],
    "spec_verify_attn_static": [_p, _i32, _i32p, _i32p, _p, _i32, ctypes.c_float, ctypes.c_float, _i32, _p, _p],
    "kv_read_status": [_p, ctypes.POINTER(ctypes.c_uint32), _i32, _p],
    "kv_stream_probe": [_p, ctypes.c_size_t, _p, ctypes.c_size_t, _p],
}

_NGRAM_SIGS = {
    "ngram_create": [ctypes.POINTER(ngram_params), ctypes.POINTER(_p)],
    "ngram_destroy": [_p],
    "ngram_observe": [_p, _i32, _i32p, _i32],
    "ngram_draft": [_p, _i32, _i32p, _i32, _i32p],
    "ngram_draft_batch": [_p, _i32, _i32p, _i32p, _i32p],
    "ngram_observe_batch": [_p, _i32, _i32p, _i32p, _i32p],
    "ngram_state": [_p, _i32, ctypes.POINTER(ctypes.c_double), _i32p, ctypes.POINTER(_i64)],
    "ngram_reset": [_p, _i32],
    "ngram_last_error": [_p],
}
_SIGS.update(_NGRAM_SIGS)

_CORE_SIGS = {
    "svcore_create": [ctypes.POINTER(svcore_params), ctypes.POINTER(_p)],
    "svcore_destroy": [_p],
    "svcore_append": [_p, _i32, _i32p, _i32p],
    "svcore_rollback": [_p, _i32, _i32],
    "svcore_seq_free": [_p, _i32],
    "svcore_seq_len": [_p, _i32, _i32p],
    "svcore_block_table": [_p, _i32, _i32p, _i32, _i32p],
    "svcore_free_blocks": [_p, _i32p],
    "svcore_codec": [_p, _p, _p, _p, _p, _p],
    "svcore_half_bits": [ctypes.c_double, ctypes.POINTER(ctypes.c_uint16), _i32p],
    "svcore_plan_verify": [_p, _i32, _i32p, _i32p, _i32, _i32, _p, _i32, _p, _p],
    "svcore_last_error": [_p],
    **_NGRAM_SIGS,
}


def _bind(lib, sigs):
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name.endswith("last_error") else ctypes.c_int
    if hasattr(lib, "kv_stream_probe_sink_bytes"):
        lib.kv_stream_probe_sink_bytes.argtypes = []
        lib.kv_stream_probe_sink_bytes.restype = ctypes.c_size_t
    return lib


def lib():
    """The loaded libsvattn.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m speculative_verify_attention_amd.build")
        _LIB = _bind(ctypes.CDLL(LIB_PATH), _SIGS)
    return _LIB


def core_lib():
    """The loaded libsvattn_core.so (HIP-free host core)."""
    global _CORE
    if _CORE is None:
        if not os.path.exists(CORE_LIB_PATH):
            raise RuntimeError(f"{CORE_LIB_PATH} is not built; run python -m speculative_verify_attention_amd.build")
        _CORE = _bind(ctypes.CDLL(CORE_LIB_PATH), _CORE_SIGS)
    return _CORE


def _arr(values):
    values = [int(x) for x in values]
    return (ctypes.c_int32 * max(1, len(values)))(*values)


def _check(rc, handle=None):
    if rc != KV_OK:
        msg = lib().kv_last_error(handle).decode() if handle else ""
        raise SvattnError(rc, msg)
    return rc


def _stream_ptr(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---- thin C-name wrappers --------------------------------------------------------------


def kv_pool_bytes(params):
    out = ctypes.c_size_t()
    _check(lib().kv_pool_bytes(ctypes.byref(params), ctypes.byref(out)))
    return out.value


def kv_record_bytes(head_dim, is_key):
    out = ctypes.c_int32()
    _check(lib().kv_record_bytes(head_dim, 1 if is_key else 0, ctypes.byref(out)))
    return out.value


def kv_create(params, stream=None):
    h = ctypes.c_void_p()
    _check(lib().kv_create(ctypes.byref(params), _stream_ptr(stream), ctypes.byref(h)))
    return h


def kv_destroy(h):
    return lib().kv_destroy(h)


def kv_append(h, seq_ids, n_new, k, v, stream=None):
    return lib().kv_append(h, len(seq_ids), _arr(seq_ids), _arr(n_new), ctypes.c_void_p(k.data_ptr()),
                           ctypes.c_void_p(v.data_ptr()), _stream_ptr(stream))


def kv_rollback(h, seq_id, n_tokens):
    return lib().kv_rollback(h, seq_id, n_tokens)


def kv_rollback_batch(h, seq_ids, n_tokens):
    return lib().kv_rollback_batch(h, len(seq_ids), _arr(seq_ids), _arr(n_tokens))


def kv_trace_events(h, before, after):
    """before/after: raw hipEvent_t handles (ints) or None."""
    return lib().kv_trace_events(h, ctypes.c_void_p(before or 0), ctypes.c_void_p(after or 0))


def kv_seq_free(h, seq_id):
    return lib().kv_seq_free(h, seq_id)


def kv_encode(h, src, is_key, dst, stream=None):
    return lib().kv_encode(h, src.shape[0], ctypes.c_void_p(src.data_ptr()), 1 if is_key else 0,
                           ctypes.c_void_p(dst.data_ptr()), _stream_ptr(stream))


def kv_workspace_bytes(h, seq_ids, n_rows, num_q_heads, window):
    out = ctypes.c_size_t()
    rc = lib().kv_workspace_bytes(h, len(seq_ids), _arr(seq_ids), _arr(n_rows), num_q_heads, window,
                                  ctypes.byref(out))
    _check(rc, h)
    return out.value


def spec_verify_attn(h, seq_ids, n_rows, q, num_q_heads, scale, softcap, window, out, workspace, stream=None):
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return lib().spec_verify_attn(h, len(seq_ids), _arr(seq_ids), _arr(n_rows), ctypes.c_void_p(q.data_ptr()),
                                  num_q_heads, float(scale), float(softcap), window,
                                  ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws_ptr), ws_bytes,
                                  _stream_ptr(stream))


def kv_workspace_bytes_valu(h, seq_ids, n_rows, num_q_heads, window):
    out = ctypes.c_size_t()
    rc = lib().kv_workspace_bytes_valu(h, len(seq_ids), _arr(seq_ids), _arr(n_rows), num_q_heads, window,
                                       ctypes.byref(out))
    _check(rc, h)
    return out.value


def spec_verify_attn_valu(h, seq_ids, n_rows, q, num_q_heads, scale, softcap, window, out, workspace, stream=None):
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return lib().spec_verify_attn_valu(h, len(seq_ids), _arr(seq_ids), _arr(n_rows), ctypes.c_void_p(q.data_ptr()),
                                       num_q_heads, float(scale), float(softcap), window,
                                       ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws_ptr), ws_bytes,
                                       _stream_ptr(stream))


def kv_append_verify_workspace_bytes(h, seq_ids, n_rows, num_q_heads, window):
    out = ctypes.c_size_t()
    rc = lib().kv_append_verify_workspace_bytes(h, len(seq_ids), _arr(seq_ids), _arr(n_rows), num_q_heads, window,
                                                ctypes.byref(out))
    _check(rc, h)
    return out.value


def kv_append_verify(h, seq_ids, n_rows, k, v, q, num_q_heads, scale, softcap, window, out, workspace, stream=None):
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return lib().kv_append_verify(h, len(seq_ids), _arr(seq_ids), _arr(n_rows), ctypes.c_void_p(k.data_ptr()),
                                  ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(q.data_ptr()), num_q_heads,
                                  float(scale), float(softcap), window, ctypes.c_void_p(out.data_ptr()),
                                  ctypes.c_void_p(ws_ptr), ws_bytes, _stream_ptr(stream))


def kv_rollback_device(h, seq_ids, n_draft, accepted, stream=None):
    return lib().kv_rollback_device(h, len(seq_ids), _arr(seq_ids), _arr(n_draft),
                                    ctypes.c_void_p(accepted.data_ptr()), _stream_ptr(stream))


def kv_sync(h):
    return lib().kv_sync(h)


def kv_seq_len(h, seq_id):
    out = ctypes.c_int32()
    _check(lib().kv_seq_len(h, seq_id, ctypes.byref(out)), h)
    return out.value


def kv_block_table(h, seq_id, cap=1 << 16):
    buf = (ctypes.c_int32 * max(1, cap))()
    n = ctypes.c_int32()
    _check(lib().kv_block_table(h, seq_id, buf, cap, ctypes.byref(n)), h)
    return list(buf[: min(cap, n.value)])


def kv_free_blocks(h):
    out = ctypes.c_int32()
    _check(lib().kv_free_blocks(h, ctypes.byref(out)), h)
    return out.value


def kv_codec(h, head_dim):
    import numpy as np

    signs = np.zeros(head_dim, dtype=np.int8)
    s = np.zeros((head_dim, head_dim), dtype=np.float32)
    lev = np.zeros(8, dtype=np.float64)
    lev16 = np.zeros(8, dtype=np.float64)
    thr = np.zeros(7, dtype=np.float64)
    _check(lib().kv_codec(h, signs.ctypes.data, s.ctypes.data, lev.ctypes.data, lev16.ctypes.data,
                          thr.ctypes.data), h)
    return signs, s, lev, lev16, thr


def spec_verify_attn_static(h, seq_ids, n_rows, q, num_q_heads, scale, softcap, window, out, stream=None):
    return lib().spec_verify_attn_static(h, len(seq_ids), _arr(seq_ids), _arr(n_rows), ctypes.c_void_p(q.data_ptr()),
                                         num_q_heads, scale, softcap, window, ctypes.c_void_p(out.data_ptr()),
                                         _stream_ptr(stream))


def kv_read_status(h, clear=False, stream=None):
    out = ctypes.c_uint32()
    _check(lib().kv_read_status(h, ctypes.byref(out), 1 if clear else 0, _stream_ptr(stream)), h)
    return out.value


def kv_stream_probe_sink_bytes():
    return lib().kv_stream_probe_sink_bytes()


def kv_stream_probe(src, sink, stream=None):
    """One streaming read of the device tensor src (its bytes) into sink."""
    _check(lib().kv_stream_probe(ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                                 ctypes.c_void_p(sink.data_ptr()), sink.numel() * sink.element_size(),
                                 _stream_ptr(stream)))


def kv_last_error(h):
    return lib().kv_last_error(h).decode()


def _check_accept(rc):
    if rc != KV_OK:
        raise SvattnError(rc, lib().spec_accept_last_error().decode())
    return rc


def spec_accept_workspace_bytes(n_draft, vocab, with_draft, temperature):
    out = ctypes.c_size_t()
    _check_accept(lib().spec_accept_workspace_bytes(len(n_draft), _arr(n_draft), vocab, int(bool(with_draft)),
                                                    float(temperature), ctypes.byref(out)))
    return out.value


def spec_accept(n_draft, target_logits, draft_logits, draft_tokens, uniforms, temperature, out_accepted,
                out_token, workspace, stream=None):
    def ptr(t):
        return ctypes.c_void_p(t.data_ptr() if t is not None else 0)

    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return lib().spec_accept(len(n_draft), _arr(n_draft), target_logits.shape[-1], ptr(target_logits),
                             ptr(draft_logits), ptr(draft_tokens), ptr(uniforms), float(temperature),
                             ptr(out_accepted), ptr(out_token), ptr(workspace), ws_bytes, _stream_ptr(stream))


def accept(n_draft, target_logits, draft_tokens, uniforms, temperature, draft_logits=None, workspace=None,
           stream=None):
    """Acceptance of drafts (argument marshalling for spec_accept).  Returns
    (accepted, token) as device int32 tensors of len(n_draft)."""
    import torch

    n_draft = [int(x) for x in n_draft]
    rows_t, rows_d = sum(n_draft) + len(n_draft), sum(n_draft)
    dev = target_logits.device
    if target_logits.dtype != torch.float32 or target_logits.dim() != 2 or target_logits.shape[0] != rows_t:
        raise ValueError(f"target_logits must be float32 [{rows_t}, vocab]")
    if not target_logits.is_contiguous():
        raise ValueError("target_logits must be contiguous")
    vocab = target_logits.shape[1]
    if draft_logits is not None and (draft_logits.dtype != torch.float32 or tuple(draft_logits.shape) != (rows_d, vocab)
                                     or not draft_logits.is_contiguous()):
        raise ValueError(f"draft_logits must be contiguous float32 [{rows_d}, {vocab}]")
    if draft_tokens.dtype != torch.int32 or draft_tokens.numel() != rows_d:
        raise ValueError(f"draft_tokens must be int32 [{rows_d}]")
    if uniforms.dtype != torch.float32 or uniforms.numel() != rows_t:
        raise ValueError(f"uniforms must be float32 [{rows_t}]")
    need = spec_accept_workspace_bytes(n_draft, vocab, draft_logits is not None, temperature)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    acc = torch.empty(len(n_draft), dtype=torch.int32, device=dev)
    tok = torch.empty(len(n_draft), dtype=torch.int32, device=dev)
    _check_accept(spec_accept(n_draft, target_logits, draft_logits, draft_tokens.contiguous(), uniforms.contiguous(),
                              temperature, acc, tok, workspace, stream))
    return acc, tok


# ---- convenience wrapper ---------------------------------------------------------------


class KVCache:
    """One layer's cache: a handle plus the torch tensor owning its pool."""

    def __init__(self, num_kv_heads, head_dim, num_blocks, max_seqs, max_blocks_per_seq, fmt, alloc_seed=0,
                 codec_seed=0, device="cuda", stream=None, ring_window=0):
        import torch

        self.num_kv_heads, self.head_dim, self.fmt = num_kv_heads, head_dim, fmt
        self.ring_window = ring_window
        self.params = kv_params(num_kv_heads, head_dim, KV_BLOCK_SIZE, num_blocks, max_seqs, max_blocks_per_seq,
                                fmt, ring_window, alloc_seed, codec_seed, None, 0)
        nbytes = kv_pool_bytes(self.params)
        self.pool = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.params.pool = self.pool.data_ptr()
        self.params.pool_bytes = nbytes
        self.handle = kv_create(self.params, stream)
        self._ws = None

    def close(self):
        if self.handle:
            kv_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check_rows(self, name, t, rows, width, dtype):
        import torch

        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA tensor")
        if t.dtype != dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dtype} tensor")
        if t.dim() != 3 or t.shape[0] < rows or t.shape[1] != width or t.shape[2] != self.head_dim:
            raise ValueError(f"{name} must have shape [>= {rows}, {width}, {self.head_dim}], got {tuple(t.shape)}")

    def append(self, seq_ids, n_new, k, v, stream=None):
        import torch

        dt = torch.bfloat16 if self.fmt == KV_BF16 else torch.float32
        rows = int(sum(n_new))
        for name, t in (("k", k), ("v", v)):
            self._check_rows(name, t, rows, self.num_kv_heads, dt)
        return _check(kv_append(self.handle, seq_ids, n_new, k, v, stream), self.handle)

    def rollback(self, seq_id, n_tokens):
        return _check(kv_rollback(self.handle, seq_id, n_tokens), self.handle)

    def rollback_batch(self, seq_ids, n_tokens):
        return _check(kv_rollback_batch(self.handle, seq_ids, n_tokens), self.handle)

    def trace_events(self, before, after):
        return _check(kv_trace_events(self.handle, before, after), self.handle)

    def seq_free(self, seq_id):
        return _check(kv_seq_free(self.handle, seq_id), self.handle)

    def seq_len(self, seq_id):
        return kv_seq_len(self.handle, seq_id)

    def block_table(self, seq_id):
        return kv_block_table(self.handle, seq_id)

    def free_blocks(self):
        return kv_free_blocks(self.handle)

    def workspace_bytes(self, seq_ids, n_rows, num_q_heads, window=0):
        return kv_workspace_bytes(self.handle, seq_ids, n_rows, num_q_heads, window)

    def workspace(self, seq_ids, n_rows, num_q_heads, window=0):
        import torch

        need = max(256, self.workspace_bytes(seq_ids, n_rows, num_q_heads, window))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.pool.device)
        return self._ws

    def verify(self, seq_ids, n_rows, q, num_q_heads, scale, softcap=0.0, window=0, out=None, workspace=None,
               stream=None):
        import torch

        rows = int(sum(n_rows))
        self._check_rows("q", q, rows, num_q_heads, torch.float32)
        if out is None:
            out = torch.empty_like(q)
        self._check_rows("out", out, rows, num_q_heads, torch.float32)
        if workspace is None:
            workspace = self.workspace(seq_ids, n_rows, num_q_heads, window)
        _check(spec_verify_attn(self.handle, seq_ids, n_rows, q, num_q_heads, scale, softcap, window, out,
                                workspace, stream), self.handle)
        return out

    def verify_valu(self, seq_ids, n_rows, q, num_q_heads, scale, softcap=0.0, window=0, out=None, workspace=None,
                    stream=None):
        """verify() with the products on the vector ALUs (spec_verify_attn_valu;
        bf16 caches at head_dim 64 and 128): the measurement twin of verify()."""
        import torch

        rows = int(sum(n_rows))
        self._check_rows("q", q, rows, num_q_heads, torch.float32)
        if out is None:
            out = torch.empty_like(q)
        self._check_rows("out", out, rows, num_q_heads, torch.float32)
        if workspace is None:
            need = max(256, kv_workspace_bytes_valu(self.handle, seq_ids, n_rows, num_q_heads, window))
            workspace = torch.empty(need, dtype=torch.uint8, device=self.pool.device)
        _check(spec_verify_attn_valu(self.handle, seq_ids, n_rows, q, num_q_heads, scale, softcap, window, out,
                                     workspace, stream), self.handle)
        return out

    def verify_static(self, seq_ids, n_rows, q, num_q_heads, scale, softcap=0.0, window=0, out=None, stream=None):
        """verify() on the library's fixed per-device scratch: no workspace, no
        allocation by the call (out=None allocates the output here, in Python)."""
        import torch

        rows = int(sum(n_rows))
        self._check_rows("q", q, rows, num_q_heads, torch.float32)
        if out is None:
            out = torch.empty_like(q)
        self._check_rows("out", out, rows, num_q_heads, torch.float32)
        _check(spec_verify_attn_static(self.handle, seq_ids, n_rows, q, num_q_heads, float(scale), float(softcap),
                                       window, out, stream), self.handle)
        return out

    def append_verify(self, seq_ids, n_rows, k, v, q, num_q_heads, scale, softcap=0.0, window=0, out=None,
                      workspace=None, stream=None):
        """kv_append of the verified rows' K/V, then verify them: one call
        (for the plain formats the attention kernel writes the rows itself)."""
        import torch

        rows = int(sum(n_rows))
        dt = torch.bfloat16 if self.fmt == KV_BF16 else torch.float32
        for name, t in (("k", k), ("v", v)):
            self._check_rows(name, t, rows, self.num_kv_heads, dt)
        self._check_rows("q", q, rows, num_q_heads, torch.float32)
        if out is None:
            out = torch.empty_like(q)
        self._check_rows("out", out, rows, num_q_heads, torch.float32)
        if workspace is None:
            need = max(256, kv_append_verify_workspace_bytes(self.handle, seq_ids, n_rows, num_q_heads, window))
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty(need, dtype=torch.uint8, device=self.pool.device)
            workspace = self._ws
        _check(kv_append_verify(self.handle, seq_ids, n_rows, k, v, q, num_q_heads, scale, softcap, window, out,
                                workspace, stream), self.handle)
        return out

    def append_verify_workspace_bytes(self, seq_ids, n_rows, num_q_heads, window=0):
        return kv_append_verify_workspace_bytes(self.handle, seq_ids, n_rows, num_q_heads, window)

    def rollback_device(self, seq_ids, n_draft, accepted, stream=None):
        """Roll back n_draft[i] - accepted[i] positions, accepted being a
        device int32 tensor (spec_accept's output): no host round trip."""
        import torch

        if (not isinstance(accepted, torch.Tensor) or accepted.device.type != "cuda" or accepted.dtype != torch.int32
                or not accepted.is_contiguous() or accepted.numel() < len(seq_ids)):
            raise ValueError("accepted must be a contiguous CUDA int32 tensor with an entry per sequence")
        return _check(kv_rollback_device(self.handle, seq_ids, n_draft, accepted, stream), self.handle)

    def sync(self):
        """Apply pending device rollbacks to the host state (waits for them)."""
        return _check(kv_sync(self.handle), self.handle)

    def encode(self, src, is_key, dst=None, stream=None):
        import torch

        if dst is None:
            dst = torch.empty((src.shape[0], kv_record_bytes(self.head_dim, is_key)), dtype=torch.uint8,
                              device=src.device)
        _check(kv_encode(self.handle, src, is_key, dst, stream), self.handle)
        return dst

    def codec(self):
        return kv_codec(self.handle, self.head_dim)

    def read_status(self, clear=False, stream=None):
        """The device status word (bit 0: a norm saturated at 65504)."""
        return kv_read_status(self.handle, clear, stream)


class NgramDrafter:
    """The n-gram self-drafter (include/svdraft.h): host-side, so it runs from
    either library; ``lib`` defaults to libsvattn.so."""

    def __init__(self, max_seqs, max_drafts=4, ema_tau=0.1, ema_threshold=0.5, lib=None):
        self.lib = lib or globals()["lib"]()
        self.max_drafts = max_drafts
        p = ngram_params(max_seqs, max_drafts, ema_tau, ema_threshold)
        self.h = ctypes.c_void_p()
        rc = self.lib.ngram_create(ctypes.byref(p), ctypes.byref(self.h))
        if rc != KV_OK:
            raise SvattnError(rc, "bad drafter parameters")

    def close(self):
        if self.h:
            self.lib.ngram_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, rc):
        if rc != KV_OK:
            raise SvattnError(rc, self.lib.ngram_last_error(self.h).decode())

    def observe(self, seq, tokens):
        tokens = [int(t) for t in tokens]
        self._check(self.lib.ngram_observe(self.h, seq, _arr(tokens), len(tokens)))

    def draft(self, seq):
        out = (ctypes.c_int32 * self.max_drafts)()
        n = ctypes.c_int32()
        self._check(self.lib.ngram_draft(self.h, seq, out, self.max_drafts, ctypes.byref(n)))
        return list(out[: n.value])

    def draft_batch(self, seqs):
        out = (ctypes.c_int32 * max(1, len(seqs) * self.max_drafts))()
        n = (ctypes.c_int32 * max(1, len(seqs)))()
        self._check(self.lib.ngram_draft_batch(self.h, len(seqs), _arr(seqs), out, n))
        return [list(out[i * self.max_drafts: i * self.max_drafts + n[i]]) for i in range(len(seqs))]

    def observe_batch(self, seqs, token_lists):
        flat = [int(t) for ts in token_lists for t in ts]
        self._check(self.lib.ngram_observe_batch(self.h, len(seqs), _arr(seqs), _arr([len(t) for t in token_lists]),
                                                 _arr(flat)))

    def state(self, seq):
        ema, en, seen = ctypes.c_double(), ctypes.c_int32(), ctypes.c_int64()
        self._check(self.lib.ngram_state(self.h, seq, ctypes.byref(ema), ctypes.byref(en), ctypes.byref(seen)))
        return ema.value, bool(en.value), seen.value

    def reset(self, seq):
        self._check(self.lib.ngram_reset(self.h, seq))
