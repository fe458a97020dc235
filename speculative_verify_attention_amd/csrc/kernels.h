// kernels.h - launch arguments and host launchers of the gfx950 kernels.
// Arguments travel by value in the kernel-argument segment, so the host's
// values are captured when a launch is enqueued: no staging buffers, no
// host-to-device copies on the step path.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace svattn {

// ---- pool layout -------------------------------------------------------------
//
// One block holds 256 token positions of every kv head; inside a block each
// head's K region is followed by the other heads' K regions, then the V
// regions.  The plain formats store each 32-token sub-tile in the order the
// attention kernel's MFMA operands consume it, so that every wave-wide load
// reads 1 KiB of contiguous memory (d = head_dim, sub-tile tokens m = 0..31):
//  BF16 K sub-tile: [d/16][2][32][8]: (kk, h, m, e) = K[m][16kk + 8h + e]
//  BF16 V sub-tile: [2][d/32][2][32][8]:
//                   (v, dt, h, r, e) = V[16v + 8(e>>2) + 4h + (e&3)][32dt + r]
//  FP32 K sub-tile: [d/8][2][32][4]: (kq, h, m, e) = K[m][(d/2)h + 4kq + e]
//  FP32 V sub-tile: [4][d/32][2][32][4]: (uq, dt, h, r, e) = V[8uq + 4h + e][32dt + r]
//  TQ3: per head, 8 sub-tiles of 32 tokens, each of 28 d + 192 bytes:
//    K codes [d/64][64 lanes][16 B]: lane 32h + m, its 16 bytes = 4 k-steps
//      kk = 4j..4j+3, 4 bytes each = nibbles of dims 16kk + 8h + e
//      (e = 0..7, nibble e at bits 4e), nibble = code | sign << 3;
//    V codes [d/64][64 lanes][12 B]: lane 32h + r, bytes 0-5 for d-tile 2j,
//      6-11 for 2j+1; in each 48-bit field 16 codes at bits 3q, q = 0..15,
//      q <-> token 16(q>>3) + 8((q&7)>>2) + 4h + (q&3), dimension 32dt + r;
//    scales [2 halves][3 fields][16] fp16: fields K norm, K residual norm,
//      V norm; half h, index i <-> token 8(i>>2) + 4h + (i&3).
struct PoolLayout {
  int32_t fmt, hkv, d;
  int64_t block_bytes;
  int64_t k_off, v_off;  // FP32/BF16 regions (TQ3: one region of 8 sub-tiles per head)
};

// Element offset of (token slot j in 0..255, dimension d) inside one head's
// K or V region of a block, for the plain formats.
__host__ __device__ inline int64_t plain_k_index(int fmt, int D, int j, int d) {
  const int64_t sb = j >> 5, m = j & 31;
  if (fmt == 1) return sb * 32 * D + (((d >> 4) * 2 + ((d >> 3) & 1)) * 32 + m) * 8 + (d & 7);
  const int h = d / (D / 2), r = d % (D / 2);
  return sb * 32 * D + (((r >> 2) * 2 + h) * 32 + m) * 4 + (r & 3);
}
__host__ __device__ inline int64_t plain_v_index(int fmt, int D, int j, int d) {
  const int64_t sb = j >> 5;
  const int t = j & 31, dt = d >> 5, dr = d & 31;
  if (fmt == 1) {
    const int v = t >> 4, rest = t & 15, h = (rest >> 2) & 1, e = 4 * (rest >> 3) + (rest & 3);
    return sb * 32 * D + (((v * (D / 32) + dt) * 2 + h) * 32 + dr) * 8 + e;
  }
  const int uq = t >> 3, h = (t >> 2) & 1, e = t & 3;
  return sb * 32 * D + (((uq * (D / 32) + dt) * 2 + h) * 32 + dr) * 4 + e;
}


// Bytes of one 32-token TQ3 sub-tile of one head.
__host__ __device__ constexpr int tq3_sub_bytes(int d) { return 28 * d + 192; }
// Byte (and nibble) of key dimension i of sub-tile token m.
__host__ __device__ inline int tq3_k_byte(int d, int m, int i, int* nibble) {
  const int kk = i >> 4, h = (i >> 3) & 1, e = i & 7;
  *nibble = e & 1;
  return (kk >> 2) * 1024 + (32 * h + m) * 16 + (kk & 3) * 4 + (e >> 1);
}
// Byte offset of the 48-bit V field holding dimension i of token t (0..31),
// and the code's bit position inside that field.
__host__ __device__ inline int tq3_v_field(int d, int t, int i, int* bit) {
  const int v = t >> 4, h = (t >> 2) & 1, q = 8 * v + 4 * ((t >> 3) & 1) + (t & 3);
  const int dt = i >> 5, r = i & 31;
  *bit = 3 * q;
  return 16 * d + (dt >> 1) * 768 + (32 * h + r) * 12 + (dt & 1) * 6;
}
// Byte offset of scale field f (0 K norm, 1 K residual norm, 2 V norm) of token t.
__host__ __device__ inline int tq3_scale_byte(int d, int t, int f) {
  const int h = (t >> 2) & 1, i = 4 * (t >> 3) + (t & 3);
  return 28 * d + (h * 3 + f) * 32 + i * 2;
}

PoolLayout make_layout(int fmt, int hkv, int d);

// ---- block-table update ------------------------------------------------------
constexpr int kMaxTableUpdates = 256;
struct TableUpdateArgs {
  int32_t* table;
  int32_t count;
  int32_t index[kMaxTableUpdates];
  int32_t block[kMaxTableUpdates];
};
hipError_t launch_table_update(const TableUpdateArgs& a, hipStream_t s);

// ---- device-side rollback ------------------------------------------------------
// roll[seq] += clamp(n_draft[i] - accepted[i], 0, n_draft[i]) for each entry:
// the lengths the kernels use are the host's minus roll[seq] until the host
// reads roll back and applies it (then roll is cleared).
constexpr int kMaxRollback = 256;
struct RollbackArgs {
  int32_t* roll;            // [max_seqs]
  const int32_t* accepted;  // device [count], this launch's entries
  int32_t count;
  int32_t seq[kMaxRollback];
  int32_t n_draft[kMaxRollback];
};
hipError_t launch_rollback(const RollbackArgs& a, hipStream_t s);
hipError_t launch_fill_zero(int32_t* p, int32_t n, hipStream_t s);

// ---- append (slice-update of new positions into their blocks) ----------------
constexpr int kMaxAppendSegs = 96;
struct AppendArgs {
  uint8_t* pool;
  const int32_t* table;
  const void* k;  // [rows][hkv][d] (this launch's rows)
  const void* v;
  PoolLayout lay;
  int32_t max_bps;
  int32_t n_segs;
  int32_t total_units;             // grid size / hkv: rows (plain) or 64-token groups (TQ3)
  int32_t unit0[kMaxAppendSegs + 1];  // prefix over segments of their units
  int32_t seq[kMaxAppendSegs];
  int32_t pos0[kMaxAppendSegs];
  int32_t n[kMaxAppendSegs];
  int32_t row0[kMaxAppendSegs];    // first source row of the segment
  int32_t keep[kMaxAppendSegs];    // positions below this are not stored (ring caches)
  // pending device rollbacks: a segment starts at pos0 - roll[seq] (null: none);
  // with them, TQ3 segments carry one spare sub-tile unit for the unknown alignment
  const int32_t* roll;
  // TQ3 codec (device constants in the pool's metadata region)
  const int8_t* signs;  // [d]
  const float* s_t;     // S transposed: [d][d], s_t[j*d + i] = S[i][j]
  double thr[7];
  double lev16[8];
  uint32_t* status;     // bit 0: a norm saturated at 65504
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);

// ---- pure encode --------------------------------------------------------------
struct EncodeArgs {
  const float* src;  // [n][d]
  uint8_t* dst;      // [n][record bytes]
  int64_t n;
  int32_t d, is_key;
  const int8_t* signs;
  const float* s_t;
  double thr[7];
  double lev16[8];
  uint32_t* status;
};
hipError_t launch_encode(const EncodeArgs& a, hipStream_t s);

// ---- verify attention ------------------------------------------------------------

// A call's work is cut into chunks of consecutive tiles of one (sequence, kv
// head) pair; workgroup w takes one chunk.  Sequence i's pairs are split into
// ksplit[i] chunks each, and its workgroups are wg_base[i] .. wg_base[i+1]-1
// (kv head major).  A pair split into more than one chunk leaves one partial
// slot per chunk (slot index = workgroup index) for the merge.
struct AttnArgs {
  const uint8_t* pool;
  const int32_t* table;
  const int8_t* signs;  // TQ3: rotation signs D (merge applies Pi^T)
  const float* q;    // [rows][hq][d] (TQ3: q' = Pi q)
  const float* q2;   // TQ3: q'' = S Pi q
  float* out;        // [rows][hq][d]
  float* part;       // partial slots
  PoolLayout lay;
  // g: query heads of a kv head this launch serves (one head slice);
  // query head of column head j of kv head h = h * gq + head0 + j
  int32_t hq, g, gq, head0, max_bps, window;
  float scale;       // multiplies <q, k>
  float softcap;     // 0 = off
  float inv_softcap;
  float qjl_coef;    // TQ3: sqrt(pi/2) / d
  float inv_sqrt_d;  // TQ3
  // TQ3 scores in log2 units: score = q1_mul (n16 <q', c16> + g16 <q2_mul q'', b>),
  // q2_mul applied before q'' is rounded to fp16 (it keeps q'' and its
  // low-order part within the normal fp16 range)
  float q1_mul;      // scale * log2(e) / sqrt(d)
  float q2_mul;      // sqrt(pi/2) / sqrt(d)
  float cap_l2;      // softcap * log2(e) (TQ3 scores are in log2 units)
  float inv_cap_l2;  // 1 / cap_l2
  int32_t n_seqs;
  int32_t n_wg;
  int32_t slot_stride;    // floats per partial slot
  int32_t rpad;           // padded rows per slot (32 * NCT)
  int32_t force_partial;  // 1: every pair goes through the merge
  int32_t tile_keys;      // keys per tile (tile_keys(fmt, d))
  uint16_t lev16_bits[8];
  // pending device rollbacks: sequence s has len[s] - roll[seq[s]] positions
  // (null: none pending)
  const int32_t* roll;
  // fused append (plain formats): the K/V rows of the verified rows, in the
  // pool's element type, [rows][hkv][d] in query-row order; the workgroups
  // whose chunk holds a row write it into the pool before reading the chunk.
  // new_k == null: no append.
  const void* new_k;
  const void* new_v;
  int32_t seq[kMaxAttnSeqs];
  int32_t len[kMaxAttnSeqs];
  int32_t qrow0[kMaxAttnSeqs];
  int32_t nrows[kMaxAttnSeqs];
  int32_t ksplit[kMaxAttnSeqs];
  int32_t wg_base[kMaxAttnSeqs + 1];
};

struct QPrepArgs {
  const float* q;   // [rows][hq][d]
  float* q1;        // Pi q
  float* q2;        // S Pi q
  const int8_t* signs;
  const float* s_t;
  int32_t n_vec, d;
};

// ---- acceptance of drafts ------------------------------------------------------
//
// Rows: the target rows of all sequences (sum of n+1), then the draft rows
// (sum of n).  A row is cut into chunks of kAcceptChunk logits; the first
// kernel reduces every (row, chunk); the second decides each sequence (every
// workgroup of a sequence takes the same decision from the row statistics)
// and sums the final draw's weights over one chunk; the third draws the token.
constexpr int kMaxAcceptSeqs = 128;
constexpr int kAcceptChunk = 4096;

// Per-sequence draw handed from the decide kernel to the pick kernel.
struct AcceptPlan {
  int32_t mode;    // 0 token already written (greedy), 1 draw from the weights
  int32_t row_t;   // target row of the weights
  int32_t row_q;   // draft row (-1: none)
  int32_t tok_q;   // point-mass draft token whose mass is removed (-1: none)
  float m_t, is_t; // target row max and 1 / sum of exp((l - max) / T)
  float m_q, is_q; // draft row, likewise
  float u;         // uniform of the draw
  int32_t pad[3];
};

struct AcceptArgs {
  const float* target;      // [rows_t][vocab]
  const float* draft;       // [rows_d][vocab] or null (point-mass drafts)
  const int32_t* drafts;    // [rows_d]
  const float* u;           // [rows_t]
  int32_t* out_acc;         // [n_seqs] (this group's first sequence at index seq0)
  int32_t* out_tok;
  float4* stats;            // [rows_t + rows_d][nch]: max, sum, argmax bits, -
  AcceptPlan* plan;         // [n_seqs]
  float* fsum;              // [n_seqs][nch] chunk sums of each draw's weights
  float inv_t;              // 1 / temperature, 0 = greedy
  int32_t vocab, nch, rows_t, rows_d;
  int32_t seq0, count;      // this launch group's sequences
  int32_t n[kMaxAcceptSeqs];   // drafts of each sequence
  int32_t t0[kMaxAcceptSeqs];  // first target row
  int32_t d0[kMaxAcceptSeqs];  // first draft row (relative to rows_t)
};

// ---- fixed device scratch (spec_verify_attn_static) ------------------------------------
// 32 MiB per device, held until the process ends; the device address of the
// calling thread's current device (resolved on first use with that device
// current).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(void** out);

// ---- streaming-read probe ------------------------------------------------------------
// Workgroups of the probe (one per compute unit); the sink holds one word each.
constexpr int kProbeWorkgroups = 256;
hipError_t launch_stream_probe(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);

static_assert(sizeof(AttnArgs) <= 4096, "kernel arguments must fit the 4 KiB argument segment");
static_assert(sizeof(AcceptArgs) <= 4096, "kernel arguments must fit the 4 KiB argument segment");
static_assert(sizeof(AppendArgs) <= 4096, "kernel arguments must fit the 4 KiB argument segment");
static_assert(sizeof(TableUpdateArgs) <= 4096, "kernel arguments must fit the 4 KiB argument segment");

hipError_t launch_attn(const AttnArgs& a, int nct, hipStream_t s);
hipError_t launch_merge(const AttnArgs& a, int nct, hipStream_t s);
// TQ3: the query rotation, and the partial kernel (two-part (hi + lo) fp16
// operands).
hipError_t launch_qprep(const QPrepArgs& a, hipStream_t s);
// One launch that encodes a TQ3 append (a) and rotates the queries (q).
hipError_t launch_append_qprep(const AppendArgs& a, const QPrepArgs& q, hipStream_t s);
hipError_t launch_attn_tq3(const AttnArgs& a, int nct, hipStream_t s);
// The partial kernel with its products on the vector ALUs (bf16 caches,
// d = 64 or 128, at most kValuMaxCols query columns: plans with that cap).
constexpr int kValuMaxCols = 20;
hipError_t launch_attn_valu(const AttnArgs& a, hipStream_t s);
// Acceptance: row statistics over every row (once per call), then decide and
// draw for one group of up to kMaxAcceptSeqs sequences.
hipError_t launch_accept_stats(const AcceptArgs& a, hipStream_t s);
hipError_t launch_accept_group(const AcceptArgs& a, hipStream_t s);

}  // namespace svattn
