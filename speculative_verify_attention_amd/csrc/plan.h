// plan.h - host planning of a verify call, HIP-free: how a call's
// (sequence, kv head) pairs are cut into chunks of tiles, which workgroup
// takes which chunk, where each chunk's partial result goes, and how much
// workspace the call needs.  The kernels recompute each workgroup's chunk
// from the same tables (ksplit, wg_base) and the lengths they read on the
// device; check_plan states what they rely on.
//
// AX Engine page, "Core Technical Architecture & Methods": the verify step
// attends 1 + k query rows of each sequence to that sequence's cache;
// SwiftLM page, long-context passage: contexts up to 100K tokens, hence the
// split of one pair over many workgroups and a merge of their partials.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "kvcore.h"

namespace svattn {

// Sequences one attention launch takes (its per-sequence fields travel in the
// kernel arguments).
#ifndef SVATTN_MAX_ATTN_SEQS
#define SVATTN_MAX_ATTN_SEQS 128
#endif
constexpr int kMaxAttnSeqs = SVATTN_MAX_ATTN_SEQS;

// Workgroups a verify call is split into (one round on 256 compute units at
// one workgroup per CU); build-time constants so variants can be measured.
#ifndef SVATTN_WG_PER_CALL
#define SVATTN_WG_PER_CALL 256
#endif
#ifndef SVATTN_WG_PER_CALL_D256
#define SVATTN_WG_PER_CALL_D256 256
#endif

// Keys per attention tile (one wavefront iteration): 16 KiB of bf16 K and V
// at d <= 128, one 32-key sub-tile otherwise.
constexpr int tile_keys(int fmt, int d) { return fmt == 1 ? 32 * (128 / d > 1 ? 128 / d : 1) : 32; }

// Workspace pieces are 256-byte aligned.
constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct VerifyLaunch {
  int first, count;  // sequences [first, first+count) of the call, in kernel order
  int n_wg;
  int64_t slot0;     // first partial slot of this launch
  std::vector<int32_t> ksplit, wg_base;
};

// Query columns of a (sequence, kv head) pair are rows x group heads.  More
// than 64 (two 32-column groups) are served by splitting the group's heads
// into hs slices of gs heads each, gs the largest divisor of the group with
// max rows x gs <= 64; each slice is its own set of launches over the same
// keys, with its own partial slots.
struct VerifyPlan {
  int nct = 1, rpad = 32;
  int hs = 1, gs = 1;          // head slices and query heads per slice
  std::vector<int> order;      // call index of the i-th sequence handed to the kernels
  std::vector<int32_t> qrow0;  // first query/output row of each call index
  int64_t slot_stride = 0, slots = 0, rows = 0;
  size_t part_bytes = 0, q_bytes = 0, total = 0;
  std::vector<VerifyLaunch> launches;
};

// Lengths a verify call plans with.  pend (max_seqs entries, or null) holds
// the device rollbacks not yet read back: the host's length (plus the rows a
// fused append adds first) is an upper bound of what the kernels will see,
// minus pend a lower bound.  Tiles are planned from the lower bound's window
// start to the upper bound's end; the kernels cut their chunks to the
// lengths they read on the device.
void verify_lengths(const Core& core, const int32_t* pend, int32_t seq, int32_t added, int32_t* up, int32_t* low);

// Plan a verify call: validates the arguments (status codes as
// spec_verify_attn's) and fills vp.  added: rows a fused append adds to each
// entry before the verify (null: none).  Built with SVATTN_CHECKED, every
// plan is also run through check_plan and a violation aborts.
// max_cols: the most query columns one slice may hold, 8 .. 64, or 0 for
// the matrix-core kernels' cap (mfma_max_cols); 20 for the vector-unit
// kernel.
int plan_verify(const Core& core, const int32_t* pend, int32_t n_seqs, const int32_t* seq_ids,
                const int32_t* n_rows, int32_t num_q_heads, int32_t window, const int32_t* added, VerifyPlan* vp,
                std::string* err, int max_cols = 0);

// Query columns one matrix-core workgroup holds: two 32-column groups, or
// one for the compressed format at d = 256 (whose registers and LDS hold a
// single group's query fragments).
constexpr int mfma_max_cols(int fmt, int d) { return fmt == 2 && d > 128 ? 32 : 64; }

// The invariants the kernels and the workspace layout rely on, checked from
// scratch against the call's arguments: the launch and chunk tables, the
// partial slots, the row offsets and the byte counts.  Returns "" when they
// hold, else a description of the first violation.
std::string check_plan(const Core& core, const int32_t* pend, int32_t n_seqs, const int32_t* seq_ids,
                       const int32_t* n_rows, int32_t num_q_heads, int32_t window, const int32_t* added,
                       const VerifyPlan& vp, int max_cols = 0);

}  // namespace svattn
