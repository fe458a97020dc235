/*
 * svcore.h - C entry points onto the HIP-free host core of the KV cache
 * (libsvattn_core.so; the same code is linked into libsvattn.so).
 *
 * These expose the host bookkeeping alone - block allocator, per-sequence
 * block tables, seq_len, all-or-nothing append reservation, O(1) rollback -
 * and the compressed format's codec constants, without any device.  They
 * exist so that the host logic behind kv_append / kv_rollback / kv_seq_free
 * can be exercised on a machine without a GPU.
 *
 * Behaviour and status codes are those of the matching kv_* calls in
 * svattn.h (AX Engine page, "Core Technical Architecture & Methods":
 * deterministic, synchronous block manager; slice-update appends; rollback
 * moves the length pointer only.  mlx-engine blog, prompt-caching section:
 * 256-token blocks).  Ownership: svcore_create allocates a handle that
 * svcore_destroy frees; all array arguments are host memory read or written
 * during the call only.
 */
#ifndef SVCORE_H
#define SVCORE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct svcore svcore; /* opaque */

typedef struct {
  int32_t num_kv_heads, head_dim, block_size, num_blocks, max_seqs, max_blocks_per_seq, format;
  int32_t ring_window; /* as kv_params.ring_window */
  uint64_t alloc_seed, codec_seed;
} svcore_params;

/* Create a host-only core; returns 0 or KV_EINVAL (-1) for bad parameters. */
int svcore_create(const svcore_params* p, svcore** out);
int svcore_destroy(svcore* c);
/* kv_append's reservation: all-or-nothing; 0, -1 EINVAL, -2 ENOMEM, -3 ERANGE, -4 ENOSEQ. */
int svcore_append(svcore* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new);
/* kv_rollback: 0, -1 (n < 0), -3 (n > seq_len), -4 (bad id). */
int svcore_rollback(svcore* c, int32_t seq, int32_t n);
/* kv_seq_free. */
int svcore_seq_free(svcore* c, int32_t seq);
int svcore_seq_len(const svcore* c, int32_t seq, int32_t* out);
/* Copy up to cap table entries; *n_owned = table entries in use (ring
 * caches: entries of released blocks read -1). */
int svcore_block_table(const svcore* c, int32_t seq, int32_t* out, int32_t cap, int32_t* n_owned);
int svcore_free_blocks(const svcore* c, int32_t* out);
/* Codec constants of a KV_TQ3 core (see kv_codec in svattn.h). */
int svcore_codec(const svcore* c, int8_t* signs, float* s_matrix, double* levels, double* levels16,
                 double* thresholds);
/* Round a double to IEEE half bits (nearest-even, saturating at 65504). */
int svcore_half_bits(double x, uint16_t* out, int32_t* saturated);
/*
 * Plan a verify call on the host-only core: the planning spec_verify_attn
 * and kv_append_verify do before they enqueue anything (AX Engine page,
 * "Core Technical Architecture & Methods": 1 + k rows per sequence checked
 * against its cache; SwiftLM page, long-context passage: a long pair is
 * split over many workgroups and their partials merged).  The plan is then
 * checked against the invariants its kernels rely on: launches of at most
 * 128 sequences, each (sequence, kv head) pair cut into non-empty chunks of
 * tiles, one partial slot per workgroup, row offsets, workspace bytes.
 * pending: max_seqs device rollbacks not yet read back (null: none); fused:
 * nonzero plans kv_append_verify (the rows are appended first).
 * summary[7] receives: column groups, launches (per head slice), partial
 * slots (per head slice), workspace bytes, partial bytes, rotated-query
 * bytes, head slices (the query heads of a kv head are split into this many
 * slices, each verified by its own launches, when rows x group heads
 * exceeds 64).  ksplit (n_seqs entries, call
 * order, or null) receives the chunks per kv head of each entry.
 * Returns 0, the status codes of spec_verify_attn's argument checks, or -5
 * when the plan breaks an invariant (svcore_last_error says which).
 */
int svcore_plan_verify(svcore* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows,
                       int32_t num_q_heads, int32_t window, const int32_t* pending, int32_t fused,
                       int64_t* summary, int32_t* ksplit);
const char* svcore_last_error(const svcore* c);

#ifdef __cplusplus
}
#endif

#endif /* SVCORE_H */
