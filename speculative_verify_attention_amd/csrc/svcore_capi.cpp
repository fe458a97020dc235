// svcore_capi.cpp - C entry points onto the HIP-free host core alone
// (include/svcore.h).  libsvattn_core.so is this file plus kvcore.cpp built
// with plain g++: the same allocator, table, rollback and codec-constant code
// that libsvattn uses, callable on a machine without a GPU.
#include "svcore.h"

#include <string>

#include "kvcore.h"
#include "plan.h"

using namespace svattn;

struct svcore {
  Core core;
  std::string err;
};

extern "C" {

int svcore_create(const svcore_params* p, svcore** out) {
  if (!p || !out) return -1;
  *out = nullptr;
  svcore* c = new svcore();
  CoreParams cp;
  cp.num_kv_heads = p->num_kv_heads;
  cp.head_dim = p->head_dim;
  cp.block_size = p->block_size;
  cp.num_blocks = p->num_blocks;
  cp.max_seqs = p->max_seqs;
  cp.max_blocks_per_seq = p->max_blocks_per_seq;
  cp.format = p->format;
  cp.ring_window = p->ring_window;
  cp.alloc_seed = p->alloc_seed;
  cp.codec_seed = p->codec_seed;
  int rc = c->core.init(cp, &c->err);
  if (rc != 0) {
    delete c;
    return rc;
  }
  *out = c;
  return 0;
}

int svcore_destroy(svcore* c) {
  delete c;
  return 0;
}

int svcore_append(svcore* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new) {
  if (!c) return -1;
  AppendPlan plan;
  int rc = c->core.plan_append(n_seqs, seq_ids, n_new, &plan, &c->err);
  if (rc != 0) return rc;
  c->core.commit_append(plan);
  return 0;
}

int svcore_rollback(svcore* c, int32_t seq, int32_t n) {
  if (!c) return -1;
  return c->core.rollback(seq, n, &c->err);
}

int svcore_seq_free(svcore* c, int32_t seq) {
  if (!c) return -1;
  return c->core.free_seq(seq, &c->err);
}

int svcore_seq_len(const svcore* c, int32_t seq, int32_t* out) {
  if (!c || !out) return -1;
  return c->core.seq_len(seq, out);
}

int svcore_block_table(const svcore* c, int32_t seq, int32_t* out, int32_t cap, int32_t* n_owned) {
  if (!c || !n_owned || cap < 0 || (cap > 0 && !out)) return -1;
  int32_t owned;
  int rc = c->core.owned(seq, &owned);
  if (rc != 0) return rc;
  const int32_t* row = c->core.table_row(seq);
  for (int i = 0; i < owned && i < cap; ++i) out[i] = row[i];
  *n_owned = owned;
  return 0;
}

int svcore_free_blocks(const svcore* c, int32_t* out) {
  if (!c || !out) return -1;
  *out = c->core.free_count();
  return 0;
}

int svcore_codec(const svcore* c, int8_t* signs, float* s_matrix, double* levels, double* levels16,
                 double* thresholds) {
  if (!c || c->core.params().format != FMT_TQ3) return -1;
  const Codec& cd = c->core.codec();
  const int d = cd.d;
  for (int i = 0; signs && i < d; ++i) signs[i] = cd.signs[i];
  for (int i = 0; s_matrix && i < d * d; ++i) s_matrix[i] = cd.s[i];
  for (int i = 0; levels && i < 8; ++i) levels[i] = cd.levels[i];
  for (int i = 0; levels16 && i < 8; ++i) levels16[i] = cd.levels16[i];
  for (int i = 0; thresholds && i < 7; ++i) thresholds[i] = cd.thresholds[i];
  return 0;
}

int svcore_half_bits(double x, uint16_t* out, int32_t* saturated) {
  if (!out) return -1;
  bool sat = false;
  *out = half_bits_rne(x, &sat);
  if (saturated) *saturated = sat ? 1 : 0;
  return 0;
}

int svcore_plan_verify(svcore* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows,
                       int32_t num_q_heads, int32_t window, const int32_t* pending, int32_t fused,
                       int64_t* summary, int32_t* ksplit) {
  if (!c || !summary) return -1;
  VerifyPlan vp;
  const int rc = plan_verify(c->core, pending, n_seqs, seq_ids, n_rows, num_q_heads, window, fused ? n_rows : nullptr,
                             &vp, &c->err);
  if (rc != 0) return rc;
  const std::string bad =
      check_plan(c->core, pending, n_seqs, seq_ids, n_rows, num_q_heads, window, fused ? n_rows : nullptr, vp);
  if (!bad.empty()) {
    c->err = "plan violates its invariants: " + bad;
    return -5;
  }
  summary[0] = vp.nct;
  summary[1] = (int64_t)vp.launches.size();
  summary[2] = vp.slots;
  summary[3] = (int64_t)vp.total;
  summary[4] = (int64_t)vp.part_bytes;
  summary[5] = (int64_t)vp.q_bytes;
  summary[6] = vp.hs;
  if (ksplit)
    for (const VerifyLaunch& L : vp.launches)
      for (int i = 0; i < L.count; ++i) ksplit[vp.order[L.first + i]] = L.ksplit[i];
  return 0;
}

const char* svcore_last_error(const svcore* c) { return c ? c->err.c_str() : "null handle"; }

}  // extern "C"
