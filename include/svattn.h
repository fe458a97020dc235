/*
 * svattn.h - C ABI of the speculative-verify attention library (libsvattn.so).
 *
 * One handle (kv_cache) is one layer's paged KV cache on one GPU.  Each
 * sequence of the cache owns 256-token blocks from a shared pool; a decode
 * step appends the k draft tokens (plus the last accepted token) of every
 * sequence, runs spec_verify_attn over the 1+k newest positions, and rolls
 * back the rejected drafts by moving seq_len only.
 *
 * Sources on the pages:
 *  - AX Engine page ("AX Engine: An LLM Inference Engine Built Exclusively
 *    for Apple Silicon M4+"), "Core Technical Architecture & Methods": up to
 *    4 drafts per step checked in one target forward; a deterministic,
 *    synchronous KV/block manager; KV grown by slice-updates into preallocated
 *    buffers; O(1) rollback that only moves the sequence-length pointer;
 *    work on dedicated streams.
 *  - AX Engine page, "Supported Model Families": dense GQA (Qwen3-4B); sliding
 *    window + full layers and a logit soft cap (Gemma4).
 *  - mlx-engine blog ("Improving LM Studio's MLX engine for agentic
 *    workflows"), model-architecture and prompt-caching sections: 512-token
 *    sliding-window local layers; caches handled in 256-token blocks; a cache
 *    must rewind to an earlier length.
 *  - SwiftLM page, TurboQuant KV-cache compression passage: keys as 3-bit
 *    Lloyd-Max codes + 1-bit QJL (4.25 bits/dim), values as 3-bit codes
 *    (3.125 bits/dim), encoded natively and dequantized inside attention.
 *
 * Conventions for every entry point:
 *  - Every function returns an int status: KV_OK (0) or a negative KV_E*
 *    code.  Arguments are validated on the host before anything is enqueued;
 *    a call that fails validation changes no state (host or device) and
 *    enqueues no work.  A call whose kernel launch fails (KV_EDEVICE) after
 *    some of its work was enqueued leaves the host state (lengths, tables,
 *    free list) unchanged too; the work already enqueued writes only
 *    positions past the committed lengths, table entries past the committed
 *    blocks, and the call's outputs, so a retry reads nothing it wrote.
 *    kv_last_error() gives a message for the last failure on a handle.
 *  - "stream" is a hipStream_t passed as void* (NULL = the null stream).  All
 *    device work of a call is enqueued on it; no call waits for the device
 *    except kv_create (once, for its constant uploads), kv_sync, and the
 *    host-side calls that first apply pending device rollbacks (see
 *    kv_rollback_device).  A handle is not thread-safe; calls on one handle
 *    must be issued from one thread and, if they use different streams,
 *    ordered by the caller.
 *  - "host" pointer arguments are read during the call only.  "device"
 *    pointers must stay valid until the enqueued work has finished.
 *  - Device faults are not detected synchronously; a sticky HIP error seen at
 *    the start of a later call is returned as KV_EDEVICE.
 */
#ifndef SVATTN_H
#define SVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KV_OK 0
#define KV_EINVAL (-1)  /* malformed argument (sizes, pointers, formats) */
#define KV_ENOMEM (-2)  /* the pool has too few free blocks, or a buffer is too small */
#define KV_ERANGE (-3)  /* a length out of range (rollback beyond seq_len, table full) */
#define KV_ENOSEQ (-4)  /* sequence id outside [0, max_seqs) */
#define KV_EDEVICE (-5) /* a HIP runtime call failed */

/* Storage format of the cached K and V. */
#define KV_FP32 0 /* float32 keys and values */
#define KV_BF16 1 /* bfloat16 keys and values */
#define KV_TQ3 2  /* compressed: see kv_encode */

#define KV_BLOCK_SIZE 256 /* token positions per block (fixed) */
#define KV_MAX_ROWS 8     /* query rows per sequence per verify call (1 + k) */

typedef struct kv_cache kv_cache; /* opaque */

typedef struct {
  int32_t num_kv_heads;       /* Hkv >= 1 */
  int32_t head_dim;           /* d: 64, 128 or 256 */
  int32_t block_size;         /* must be KV_BLOCK_SIZE */
  int32_t num_blocks;         /* blocks in the pool, >= 1 */
  int32_t max_seqs;           /* sequence ids are 0 .. max_seqs-1 */
  int32_t max_blocks_per_seq; /* table width: positions < 256 * this */
  int32_t format;             /* KV_FP32, KV_BF16 or KV_TQ3 */
  int32_t ring_window;        /* 0: plain cache; W > 0: ring cache for window layers (below) */
  uint64_t alloc_seed;        /* free-list order: 0 = identity, else a SplitMix64 Fisher-Yates shuffle */
  uint64_t codec_seed;        /* KV_TQ3 only: seeds the rotation signs and the QJL matrix */
  void* pool;                 /* device memory owned by the caller, 256-byte aligned */
  size_t pool_bytes;          /* >= kv_pool_bytes(params) */
} kv_params;

/*
 * Bytes of device memory a pool for these parameters needs (blocks followed
 * by the library's metadata: the device block table, a status word, the
 * pending device-rollback counters and, for KV_TQ3, the codec constants).
 * p->pool and p->pool_bytes are ignored.
 *
 * Block layout.  A block holds 256 token positions of every kv head: first
 * each head's K region in head order, then each head's V region.  d =
 * head_dim; m = token within a 32-token sub-tile; a region is 8 sub-tiles.
 *  KV_BF16 (2-byte elements), per sub-tile:
 *    K as [d/16][2][32][8]:       element (kk, h, m, e) = K[m][16kk + 8h + e]
 *    V as [2][d/32][2][32][8]:    element (v, dt, h, r, e) =
 *                                 V[16v + 8(e>>2) + 4h + (e&3)][32dt + r]
 *  KV_FP32 (4-byte elements), per sub-tile:
 *    K as [d/8][2][32][4]:        element (kq, h, m, e) = K[m][(d/2)h + 4kq + e]
 *    V as [4][d/32][2][32][4]:    element (uq, dt, h, r, e) = V[8uq + 4h + e][32dt + r]
 *  (this order makes every wavefront-wide load of the attention kernel read
 *  1 KiB of contiguous memory straight into its matrix-core operands).
 *  KV_TQ3: one region per kv head, in head order, of 8 sub-tiles of 32
 *  tokens, each sub-tile 28 d + 192 bytes (3776 B at d=128, i.e. 118 B per
 *  token: 68 B of key record and 50 B of value record):
 *    K codes as [d/64][64 lanes][16 B]: lane 32h + m holds, for k-steps
 *      kk = 4j .. 4j+3 (4 bytes each), the nibbles of dimensions
 *      16kk + 8h + e (e = 0..7, nibble e at bits 4e) of token m; a nibble is
 *      code | sign_bit << 3.
 *    V codes as [d/64][64 lanes][12 B]: lane 32h + r, bytes 0-5 for d-tile
 *      2j and 6-11 for d-tile 2j+1; each 48-bit little-endian field holds 16
 *      3-bit codes at bits 3q (q = 0..15) of dimension 32 dt + r of tokens
 *      16(q>>3) + 8((q&7)>>2) + 4h + (q&3).
 *    Scales as [2 halves][3 fields][16] fp16, fields K norm n16, K residual
 *      norm g16, V norm n16; half h, index i <-> token 8(i>>2) + 4h + (i&3).
 */
int kv_pool_bytes(const kv_params* p, size_t* out);

/*
 * Ring caches (ring_window = W > 0) serve sliding-window layers (mlx-engine
 * blog, model-architecture section: 512-token local layers), whose rows
 * never look further back than W - 1 positions: a sequence keeps only the
 * blocks that hold its last W + KV_MAX_ROWS positions, so its memory stays
 * at ceil((W + KV_MAX_ROWS + 255) / 256) blocks whatever its length, and
 * the rows one verify call appends can still be verified and rolled back.
 *  - After an append to length L, blocks wholly below position
 *    max(0, L - KV_MAX_ROWS - W + 1) are released (their table entries read
 *    -1) and pushed onto the front of the free list in increasing index
 *    order before the call's new blocks are popped, so they are reused
 *    first.  Appended positions below that point are not stored.  With
 *    device rollbacks pending, L is the lower bound of the length.
 *  - A rollback (host or device) that would leave a later window reaching a
 *    released position fails with KV_ERANGE: to length L' is allowed while
 *    max(0, L' - W + 1) is at or above the first kept position.
 *  - Verify calls must pass 1 <= window <= W.
 *  - max_blocks_per_seq still bounds the length (the table is indexed by
 *    position / 256); num_blocks bounds the memory.
 */

/*
 * Create a handle over a caller-owned pool.  Every sequence starts empty.
 * Uploads the codec constants (KV_TQ3) on `stream` and waits for them.
 * The pool must outlive the handle; the handle never allocates device memory.
 * Errors: KV_EINVAL (bad params), KV_ENOMEM (pool too small), KV_EDEVICE.
 */
int kv_create(const kv_params* p, void* stream, kv_cache** out);

/* Destroy a handle (waits for nothing; the caller orders it after the last
 * enqueued call).  NULL is accepted. */
int kv_destroy(kv_cache* c);

/*
 * Append n_new[i] new token positions to sequence seq_ids[i], for i < n_seqs,
 * as one all-or-nothing reservation (AX Engine page, "Core Technical
 * Architecture & Methods": slice-update into preallocated buffers).
 *  seq_ids, n_new: host arrays of n_seqs entries; ids distinct; n_new >= 0.
 *  k, v: device arrays [sum(n_new)][num_kv_heads][head_dim], rows in the
 *    order of seq_ids; dtype float32 for KV_FP32 and KV_TQ3, bfloat16 for
 *    KV_BF16.  For KV_TQ3 the rows are encoded as they are stored (the
 *    quantize-on-append path).
 * Blocks are popped from the front of the free list as a sequence's length
 * crosses 256-token boundaries.  Errors: KV_ENOSEQ, KV_EINVAL, KV_ERANGE
 * (a table would overflow), KV_ENOMEM (not enough free blocks for the whole
 * call), KV_EDEVICE.
 */
int kv_append(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new,
              const void* k, const void* v, void* stream);

/*
 * Drop the newest n_tokens positions of a sequence: seq_len -= n_tokens, in
 * O(1), host only (AX Engine page, "Core Technical Architecture & Methods").
 * Blocks stay owned; the next append overwrites the dropped slots.
 * Errors: KV_ENOSEQ, KV_EINVAL (n_tokens < 0), KV_ERANGE (n_tokens > seq_len).
 */
int kv_rollback(kv_cache* c, int32_t seq_id, int32_t n_tokens);

/*
 * kv_rollback for several sequences in one call, all-or-nothing: every entry
 * is validated first (errors as kv_rollback; a repeated id is KV_EINVAL) and
 * nothing changes unless all are valid.  seq_ids, n_tokens: host arrays.
 */
int kv_rollback_batch(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_tokens);

/*
 * Roll sequences back on the device, from acceptance counts the device
 * produced (spec_accept's out_accepted), without a device-to-host copy: the
 * rollback the AX Engine page describes ("Core Technical Architecture &
 * Methods": O(1), the length pointer only) moved to the device so that a
 * decode step (append, verify, accept, rollback) never waits for the host.
 * Sequence seq_ids[i] loses n_draft[i] - accepted[i] positions (accepted[i]
 * clamped to [0, n_draft[i]]).
 *  seq_ids, n_draft: host arrays of n_seqs entries; ids distinct;
 *    0 <= n_draft[i] <= the sequence's length.
 *  accepted: device int32 [n_seqs].
 * Until kv_sync, the host knows each length only up to the pending amount:
 * kv_append and spec_verify_attn / kv_append_verify read the exact lengths
 * on the device (reservations cover the upper bound; blocks stay owned
 * anyway).  kv_rollback, kv_rollback_batch, kv_seq_free, kv_seq_len and
 * kv_block_table first apply the pending rollbacks (kv_sync).  Every
 * kv_rollback_device call between two syncs must use the same stream.
 * Errors: KV_ENOSEQ, KV_EINVAL, KV_ERANGE, KV_EDEVICE.
 */
int kv_rollback_device(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_draft,
                       const int32_t* accepted, void* stream);

/*
 * Apply pending device rollbacks to the host state: copies the counters from
 * the device (waiting for the stream of the last kv_rollback_device call),
 * moves the host lengths, clears the counters.  A no-op without pending
 * rollbacks.  Errors: KV_EDEVICE.
 */
int kv_sync(kv_cache* c);

/* Release every block of a sequence (pushed back onto the front of the free
 * list, first-owned block first) and reset its length to 0.  The caller must
 * not free a sequence that enqueued work still reads.  Errors: KV_ENOSEQ. */
int kv_seq_free(kv_cache* c, int32_t seq_id);

/*
 * Encode n_vecs vectors with the handle's codec (KV_TQ3 handles only): the
 * quantize step of the compressed cache on its own, without touching the
 * pool (SwiftLM page, TurboQuant KV-cache compression passage).
 *  src: device float32 [n_vecs][d].
 *  dst: device, n_vecs records of kv_record_bytes(d, is_key) bytes each:
 *    key record  = d/2 code|sign nibbles, fp16 n16, fp16 g16 (68 B at d=128);
 *    value record = 3d/8 bytes of 3-bit codes (dimension i at bits 3i..3i+2,
 *    little-endian), fp16 n16 (50 B at d=128).
 * The encoder works in double precision: n = |x|, z = sqrt(d) * Pi x / n with
 * Pi = H_d diag(D) / sqrt(d), code = number of Lloyd-Max thresholds <= z_i,
 * n16 = fp16(n); keys also r = Pi x - n16 * c16[code] / sqrt(d),
 * g16 = fp16(|r|), sign bit = [(S r)_i >= 0].
 * Errors: KV_EINVAL (not a KV_TQ3 handle, n_vecs < 0), KV_EDEVICE.
 */
int kv_encode(const kv_cache* c, int64_t n_vecs, const float* src, int32_t is_key, void* dst,
              void* stream);

/* Bytes of one kv_encode record. */
int kv_record_bytes(int32_t head_dim, int32_t is_key, int32_t* out);

/*
 * Device status bits of a handle (KV_TQ3 encoders set them; see kv_encode
 * and kv_append): KV_STATUS_NORM_SATURATED when some vector's norm (or key
 * residual norm) exceeded 65504 and was stored as 65504, the largest finite
 * fp16 value.  Reads the word after the work enqueued on `stream` so far
 * (waits for that stream), stores it in *out, and clears it first if clear
 * is non-zero (with a fill kernel, no memset).  Errors: KV_EINVAL,
 * KV_EDEVICE.
 */
#define KV_STATUS_NORM_SATURATED 1u
int kv_read_status(kv_cache* c, uint32_t* out, int32_t clear, void* stream);

/*
 * Workspace bytes spec_verify_attn needs for this call shape (same arguments
 * as spec_verify_attn).  Errors as spec_verify_attn's validation.
 */
int kv_workspace_bytes(const kv_cache* c, int32_t n_seqs, const int32_t* seq_ids,
                       const int32_t* n_rows, int32_t num_q_heads, int32_t window, size_t* out);

/*
 * Verify attention over the newest positions of each sequence: the one kernel
 * path these pages revolve around (AX Engine page, "Core Technical
 * Architecture & Methods"; SwiftLM page, speculative-decoding passage: N+1
 * positions verified at once).
 *  seq_ids, n_rows: host arrays of n_seqs entries; 1 <= n_rows[i] <=
 *    min(KV_MAX_ROWS, seq_len); row r of sequence i sits at position
 *    seq_len - n_rows[i] + r, so the rows' K/V must already be appended.
 *  q: device float32 [sum(n_rows)][num_q_heads][head_dim], rows in the order
 *    of seq_ids.  num_q_heads must be a multiple of num_kv_heads; query head
 *    h reads kv head h / (num_q_heads / num_kv_heads).  The kernels hold
 *    at most 64 query columns (rows x group heads) of a kv head at once (32
 *    for KV_TQ3 at head_dim 256); beyond that (e.g. 5 rows at a group of
 *    16) the call splits each group
 *    into the fewest equal slices of heads that fit and runs one pass of
 *    launches per slice, so the cache is read once per slice and the
 *    workspace holds one set of partials per slice.
 *  scale: multiplies <q, k>.  softcap: 0 = off, else s <- softcap *
 *    tanh(s / softcap) after scaling.  window: 0 = full, else position p sees
 *    keys j with 0 <= p - j < window.  Row p never sees keys beyond itself.
 *  out: device float32 [sum(n_rows)][num_q_heads][head_dim].
 *  workspace: device, ws_bytes >= kv_workspace_bytes(...), 256-byte aligned;
 *    it holds split-context partial results.  Calls that share a workspace
 *    must be ordered on one stream.
 * KV_TQ3: queries are rotated in the kernel path (q' = Pi q, q'' = S q'),
 * scores use the stored codes and norms, and the output is rotated back.
 * Precision: products accumulate in fp32.  KV_FP32 multiplies in fp32;
 * KV_BF16 multiplies the stored bf16 K/V by the query and by the softmax
 * weights, each carried as two bf16 parts (hi + lo, about 2^-17 relative);
 * KV_TQ3 multiplies the exact fp16 code levels and signs by fp16 parts of
 * q', q'' and the weights (two parts each, about 2^-21 relative).
 * Errors: KV_ENOSEQ, KV_EINVAL (bad arguments), KV_ERANGE (n_rows > seq_len),
 * KV_ENOMEM (workspace too small), KV_EDEVICE.
 */
int spec_verify_attn(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows,
                     const float* q, int32_t num_q_heads, float scale, float softcap,
                     int32_t window, float* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * spec_verify_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): the partial results and rotated
 * queries go to a fixed scratch array of 32 MiB per device that the library
 * owns for the life of the process.  The call allocates nothing.  The
 * scratch of a device is shared by every call on it: calls that may overlap
 * on one GPU (different streams, different handles) race, so order them
 * (one stream) or use spec_verify_attn with workspaces of their own.  The
 * scratch needs no clearing: every call writes each slot it reads.
 * Arguments and results as spec_verify_attn's.  Errors: as
 * spec_verify_attn's; KV_ENOMEM when the call needs more than 32 MiB of
 * scratch (kv_workspace_bytes gives the need).
 */
int spec_verify_attn_static(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows,
                            const float* q, int32_t num_q_heads, float scale, float softcap,
                            int32_t window, float* out, void* stream);

/*
 * spec_verify_attn with the products on the vector ALUs instead of the
 * matrix cores: a measurement aid for choosing between the two units at the
 * verify step's shapes (1 + k rows x a GQA group of query columns per kv
 * head).  The same call, result and precision (the bf16 keys and values
 * times two bf16 parts of the fp32 queries and probabilities, fp32
 * accumulation, here by packed dot products), for KV_BF16 caches at
 * head_dim 64 and 128; a kv head's columns are served 20 at a time (head
 * slices beyond).  workspace: ws_bytes >= kv_workspace_bytes_valu(...).
 * Errors: as spec_verify_attn's; KV_EINVAL for another format or head_dim.
 */
int kv_workspace_bytes_valu(const kv_cache* c, int32_t n_seqs, const int32_t* seq_ids,
                            const int32_t* n_rows, int32_t num_q_heads, int32_t window, size_t* out);
int spec_verify_attn_valu(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows,
                          const float* q, int32_t num_q_heads, float scale, float softcap,
                          int32_t window, float* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * Append the verified rows' K/V and verify them, in one call: kv_append of
 * n_rows[i] positions to each sequence followed by spec_verify_attn over
 * those same positions (AX Engine page, "Core Technical Architecture &
 * Methods": slice-update appends; SwiftLM page, speculative-decoding
 * passage: the N+1 positions verified at once).  For KV_FP32 and KV_BF16
 * the attention kernel itself writes the rows into their blocks before it
 * reads them, so the append costs no launch of its own; KV_TQ3 encodes in a
 * launch before the attention.
 *  k, v: as kv_append's, [sum(n_rows)][num_kv_heads][head_dim], rows in the
 *    order of q's rows.
 *  Everything else as spec_verify_attn's; the row positions count the
 *  appended rows (row r of sequence i sits at seq_len + r before the call).
 *  workspace: ws_bytes >= kv_append_verify_workspace_bytes(...).
 * The stored bytes and outputs equal those of kv_append followed by
 * spec_verify_attn.  Errors: the union of both calls' errors; a failed call
 * changes nothing.
 */
int kv_append_verify(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows,
                     const void* k, const void* v, const float* q, int32_t num_q_heads, float scale,
                     float softcap, int32_t window, float* out, void* workspace, size_t ws_bytes,
                     void* stream);

/* Workspace bytes of kv_append_verify for this call shape (planned with the
 * lengths after the append).  Errors as kv_append_verify's validation. */
int kv_append_verify_workspace_bytes(const kv_cache* c, int32_t n_seqs, const int32_t* seq_ids,
                                     const int32_t* n_rows, int32_t num_q_heads, int32_t window,
                                     size_t* out);

/*
 * Acceptance of the drafts after the verify forward (SwiftLM page,
 * speculative-decoding passage: rejection sampling per Leviathan et al., the
 * ratio P_target / P_draft deciding each draft and a rejected position
 * re-sampled from the corrected distribution; greedy argmax when the
 * temperature is 0).  Stateless: no handle.
 *  n_seqs, n_draft: host; n_draft[i] in [0, KV_MAX_ROWS - 1].
 *  vocab: logits per row, >= 1.
 *  target_logits: device float32 [sum(n_draft + 1)][vocab], sequences in
 *    order; row j of sequence i is the target's distribution of the j-th
 *    token after the sequence's last accepted token: rows j < n_draft[i]
 *    check draft j, row n_draft[i] gives the bonus token.
 *  draft_logits: device float32 [sum(n_draft)][vocab], or NULL when the
 *    drafts are point masses (n-gram drafts, AX Engine page, "Core Technical
 *    Architecture & Methods").  Unused when temperature is 0.
 *  draft_tokens: device int32 [sum(n_draft)]; a token outside [0, vocab) is
 *    never accepted.
 *  uniforms: device float32 [sum(n_draft + 1)] in [0, 1): entry j < n decides
 *    draft j, entry n draws the final token.  Unused when temperature is 0.
 *  temperature: 0 = greedy (accept while a draft equals the first argmax of
 *    its row); > 0: p = softmax(target / T), q = softmax(draft / T), draft j
 *    accepted iff u_j * q_j(d_j) < p_j(d_j); the first rejection draws from
 *    max(0, p_j - q_j) (a point-mass draft: p_j without its token), else the
 *    bonus is drawn from p_n; a draw returns the smallest token whose
 *    cumulative weight (tokens in index order) exceeds u_n times the total.
 *  out_accepted: device int32 [n_seqs]: accepted drafts (0 .. n_draft[i]).
 *  out_token: device int32 [n_seqs]: the token that follows them.
 *  workspace: device, >= spec_accept_workspace_bytes(...), 256-byte aligned;
 *    it holds row statistics, chunk sums and draw plans, so calls
 *    that share a workspace must not overlap (order them on one stream).
 * Arithmetic is fp32; decisions within about 1e-6 relative of a threshold may
 * differ from an exact evaluation.  The caller rolls the cache back by
 * n_draft[i] - out_accepted[i] (kv_rollback_batch, after copying the counts
 * to the host).  Errors: KV_EINVAL, KV_ENOMEM (workspace), KV_EDEVICE;
 * spec_accept_last_error() gives the message of the calling thread's last
 * failure.
 */
int spec_accept(int32_t n_seqs, const int32_t* n_draft, int32_t vocab, const float* target_logits,
                const float* draft_logits, const int32_t* draft_tokens, const float* uniforms,
                float temperature, int32_t* out_accepted, int32_t* out_token, void* workspace,
                size_t ws_bytes, void* stream);

/* Workspace bytes of spec_accept for this shape (with_draft: draft_logits
 * will be non-NULL).  Errors as spec_accept's validation. */
int spec_accept_workspace_bytes(int32_t n_seqs, const int32_t* n_draft, int32_t vocab, int32_t with_draft,
                                float temperature, size_t* out);

const char* spec_accept_last_error(void);

/*
 * Tracing: while set, every spec_verify_attn and kv_append_verify call
 * records event `before` on
 * its stream just before its first attention-partial kernel and `after` just
 * after its last one (hipEvent_t handles passed as void*, owned by the
 * caller), so that hipEventElapsedTime gives the partial kernels' time
 * without the merge.  Passing NULL for both stops the recording.
 */
int kv_trace_events(kv_cache* c, void* before, void* after);

/*
 * Streaming-read probe (measurement aid, not part of the attention path):
 * reads the `bytes` bytes at src once, one workgroup per compute unit
 * walking the buffer grid-stride with 16-byte loads (every wave 1 KiB of
 * consecutive memory per load, 16 loads in flight), and folds them into one
 * word per workgroup in sink so that no load is elided.  Its duration measures the read bandwidth that a perfect
 * single-pass reader of a cache of that size reaches on this GPU.
 *  src: device, 16-byte aligned; bytes: a multiple of 16.
 *  sink: device, at least kv_stream_probe_sink_bytes() bytes.
 * Errors: KV_EINVAL, KV_EDEVICE.
 */
int kv_stream_probe(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream);
size_t kv_stream_probe_sink_bytes(void);

/* ---- introspection (host only; touches the device only to apply pending
 * device rollbacks first) ---- */

/* Current length of a sequence.  Errors: KV_ENOSEQ. */
int kv_seq_len(const kv_cache* c, int32_t seq_id, int32_t* out);

/* Copy up to cap entries of a sequence's block table to out (host) and the
 * number of table entries in use to *n_owned (ring caches: released entries
 * read -1).  Errors: KV_ENOSEQ, KV_EINVAL. */
int kv_block_table(const kv_cache* c, int32_t seq_id, int32_t* out, int32_t cap, int32_t* n_owned);

/* Number of blocks on the free list. */
int kv_free_blocks(const kv_cache* c, int32_t* out);

/* KV_TQ3 codec constants as the library computed them (host copies; any
 * pointer may be NULL): signs[d] (+-1), s_matrix[d*d] row-major float32,
 * levels[8] (the Lloyd-Max centroids, fp64), levels16[8] (the stored fp16
 * reconstruction levels, as fp64 values), thresholds[7] (fp64).
 * Errors: KV_EINVAL (not KV_TQ3). */
int kv_codec(const kv_cache* c, int8_t* signs, float* s_matrix, double* levels,
             double* levels16, double* thresholds);

/* Message for the last failed call on this handle ("" if none). */
const char* kv_last_error(const kv_cache* c);

#ifdef __cplusplus
}
#endif

#endif /* SVATTN_H */
