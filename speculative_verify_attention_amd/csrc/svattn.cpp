// svattn.cpp - the C ABI (include/svattn.h) over the host core and the
// gfx950 kernels.  Validation happens on the host before anything is
// enqueued; the core's state changes only after every launch of a call has
// been enqueued successfully.
#include "svattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"
#include "kvcore.h"
#include "plan.h"

using namespace svattn;

struct kv_cache {
  Core core;
  PoolLayout lay;
  uint8_t* pool = nullptr;
  size_t pool_bytes = 0;
  int32_t* dtable = nullptr;   // device block table [max_seqs][max_blocks_per_seq]
  uint32_t* dstatus = nullptr; // device status word
  int32_t* droll = nullptr;    // device rollbacks not yet applied on the host [max_seqs]
  int8_t* dsigns = nullptr;    // TQ3: D
  float* ds_t = nullptr;       // TQ3: S transposed
  std::vector<int8_t> h_signs;
  std::vector<float> h_s_t;
  std::vector<uint32_t> h_zero;
  // Device rollbacks (kv_rollback_device) not yet read back: the host's
  // lengths are upper bounds, the device's are len - droll[seq], and
  // pend[seq] bounds droll[seq] from above.
  std::vector<int32_t> pend;
  std::vector<int32_t> h_roll;
  bool any_pend = false;
  hipStream_t pend_stream = nullptr;
  hipEvent_t trace_before = nullptr, trace_after = nullptr;
  std::string err;
};

namespace {

struct MetaLayout {
  size_t blocks_bytes, table_off, status_off, roll_off, signs_off, st_off, total;
};

MetaLayout meta_layout(const kv_params& p, const PoolLayout& lay) {
  MetaLayout m;
  m.blocks_bytes = (size_t)p.num_blocks * (size_t)lay.block_bytes;
  m.table_off = align_up(m.blocks_bytes);
  m.status_off = align_up(m.table_off + (size_t)p.max_seqs * p.max_blocks_per_seq * 4);
  m.roll_off = m.status_off + kAlign;
  m.signs_off = align_up(m.roll_off + (size_t)p.max_seqs * 4);
  m.st_off = m.signs_off;
  m.total = m.signs_off;
  if (p.format == KV_TQ3) {
    m.st_off = align_up(m.signs_off + (size_t)p.head_dim);
    m.total = align_up(m.st_off + (size_t)p.head_dim * p.head_dim * 4);
  }
  return m;
}

int sync_pending(kv_cache* c);
int enqueue_table_updates(kv_cache* c, const AppendPlan& plan, hipStream_t s);

// Per call entry: the pending device rollbacks of its sequence (0 for bad ids,
// which the plan rejects).
std::vector<int32_t> pending_slack(const kv_cache* c, int32_t n_seqs, const int32_t* seq_ids);

int set_err(kv_cache* c, int code, const std::string& msg) {
  if (c) c->err = msg;
  return code;
}

int check_device(kv_cache* c) {
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_err(c, KV_EDEVICE, std::string("HIP error before call: ") + hipGetErrorString(e));
  }
  return KV_OK;
}

int hip_fail(kv_cache* c, hipError_t e, const char* what) {
  return set_err(c, KV_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

CoreParams core_params(const kv_params& p) {
  CoreParams cp;
  cp.num_kv_heads = p.num_kv_heads;
  cp.head_dim = p.head_dim;
  cp.block_size = p.block_size;
  cp.num_blocks = p.num_blocks;
  cp.max_seqs = p.max_seqs;
  cp.max_blocks_per_seq = p.max_blocks_per_seq;
  cp.format = p.format;
  cp.ring_window = p.ring_window;
  cp.alloc_seed = p.alloc_seed;
  cp.codec_seed = p.codec_seed;
  return cp;
}

// ---- verify-call planning (shared by kv_workspace_bytes and spec_verify_attn) ----

void verify_lengths(const kv_cache* c, int32_t seq, int32_t added, int32_t* up, int32_t* low) {
  svattn::verify_lengths(c->core, c->pend.data(), seq, added, up, low);
}

int plan_verify(const kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows,
                int32_t num_q_heads, int32_t window, const int32_t* added, VerifyPlan* vp, std::string* err,
                int max_cols = 0) {
  return svattn::plan_verify(c->core, c->pend.data(), n_seqs, seq_ids, n_rows, num_q_heads, window, added, vp, err,
                             max_cols);
}

// The vector-unit verify's plan: at most kValuMaxCols columns per slice.
int plan_verify_valu(const kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows,
                     int32_t num_q_heads, int32_t window, VerifyPlan* vp) {
  kv_cache* cc = const_cast<kv_cache*>(c);
  const CoreParams& P = c->core.params();
  if (P.format != KV_BF16 || (P.head_dim != 64 && P.head_dim != 128)) {
    cc->err = "the vector-unit verify serves KV_BF16 caches at head_dim 64 and 128";
    return KV_EINVAL;
  }
  return plan_verify(c, n_seqs, seq_ids, n_rows, num_q_heads, window, nullptr, vp, &cc->err, kValuMaxCols);
}

}  // namespace

extern "C" {

int kv_pool_bytes(const kv_params* p, size_t* out) {
  if (!p || !out) return KV_EINVAL;
  Core probe;
  std::string err;
  kv_params q = *p;
  if (probe.init(core_params(q), &err) != KV_OK) return KV_EINVAL;
  PoolLayout lay = make_layout(p->format, p->num_kv_heads, p->head_dim);
  *out = meta_layout(*p, lay).total;
  return KV_OK;
}

int kv_record_bytes(int32_t head_dim, int32_t is_key, int32_t* out) {
  if (!out || (head_dim != 64 && head_dim != 128 && head_dim != 256)) return KV_EINVAL;
  *out = is_key ? head_dim / 2 + 4 : 3 * head_dim / 8 + 2;
  return KV_OK;
}

int kv_create(const kv_params* p, void* stream, kv_cache** out) {
  if (!p || !out) return KV_EINVAL;
  *out = nullptr;
  kv_cache* c = new kv_cache();
  std::string err;
  int rc = c->core.init(core_params(*p), &err);
  if (rc != KV_OK) {
    delete c;
    return rc;
  }
  c->lay = make_layout(p->format, p->num_kv_heads, p->head_dim);
  MetaLayout m = meta_layout(*p, c->lay);
  if (!p->pool || (reinterpret_cast<uintptr_t>(p->pool) % kAlign) != 0) {
    delete c;
    return KV_EINVAL;
  }
  if (p->pool_bytes < m.total) {
    delete c;
    return KV_ENOMEM;
  }
  if (check_device(c) != KV_OK) {
    delete c;
    return KV_EDEVICE;
  }
  c->pool = static_cast<uint8_t*>(p->pool);
  c->pool_bytes = p->pool_bytes;
  c->dtable = reinterpret_cast<int32_t*>(c->pool + m.table_off);
  c->dstatus = reinterpret_cast<uint32_t*>(c->pool + m.status_off);
  c->droll = reinterpret_cast<int32_t*>(c->pool + m.roll_off);
  c->pend.assign(p->max_seqs, 0);
  c->h_roll.assign(p->max_seqs, 0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  c->h_zero.assign(std::max<size_t>(kAlign / 4, (size_t)p->max_seqs), 0u);
  hipError_t e = hipMemcpyAsync(c->dstatus, c->h_zero.data(), kAlign, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(c->droll, c->h_zero.data(), (size_t)p->max_seqs * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && p->format == KV_TQ3) {
    const Codec& cd = c->core.codec();
    const int d = p->head_dim;
    c->dsigns = reinterpret_cast<int8_t*>(c->pool + m.signs_off);
    c->ds_t = reinterpret_cast<float*>(c->pool + m.st_off);
    c->h_signs = cd.signs;
    c->h_s_t.resize((size_t)d * d);
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) c->h_s_t[(size_t)j * d + i] = cd.s[(size_t)i * d + j];
    e = hipMemcpyAsync(c->dsigns, c->h_signs.data(), d, hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(c->ds_t, c->h_s_t.data(), (size_t)d * d * 4, hipMemcpyHostToDevice, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete c;
    return KV_EDEVICE;
  }
  *out = c;
  return KV_OK;
}

int kv_destroy(kv_cache* c) {
  delete c;
  return KV_OK;
}

}  // extern "C"

namespace {

// Enqueue a planned append (table updates, then the slice-update or
// quantize-on-append launches) without committing it to the host state.
// qp (TQ3, optional): the queries' rotation, launched together with the last
// append launch; *qp_done tells whether it was (not when nothing is stored).
int enqueue_append(kv_cache* c, const AppendPlan& plan, const std::vector<int32_t>& slack, const void* k,
                   const void* v, hipStream_t s, const QPrepArgs* qp = nullptr, bool* qp_done = nullptr) {
  if (qp_done) *qp_done = false;
  // 1. new blocks become visible in the device table
  int rc = enqueue_table_updates(c, plan, s);
  if (rc != KV_OK) return rc;
  // 2. slice-update / quantize-on-append, in launches of <= kMaxAppendSegs segments
  const CoreParams& P = c->core.params();
  // A ring cache stores nothing below its first kept block: with no device
  // rollback pending the rows are trimmed here, else the kernels skip them
  // (the true positions are known on the device only).
  std::vector<AppendSeg> stored;
  for (size_t i = 0; i < plan.segs.size(); ++i) {
    AppendSeg g = plan.segs[i];
    const int32_t keep = g.keep_first * kBlock;
    if (slack[i] == 0 && g.pos0 < keep) {
      const int32_t cut = std::min(g.n, keep - g.pos0);
      g.pos0 += cut;
      g.n -= cut;
      g.src_row0 += cut;
    }
    stored.push_back(g);
  }
  std::vector<const AppendSeg*> segs;
  for (const AppendSeg& g : stored)
    if (g.n > 0) segs.push_back(&g);
  const bool tq3 = P.format == KV_TQ3;
  for (size_t i = 0; i < segs.size();) {
    AppendArgs a;
    std::memset(&a, 0, sizeof(a));
    a.pool = c->pool;
    a.table = c->dtable;
    a.k = k;
    a.v = v;
    a.lay = c->lay;
    a.max_bps = P.max_blocks_per_seq;
    a.n_segs = 0;
    int64_t units = 0;
    while (i < segs.size() && a.n_segs < kMaxAppendSegs) {
      const AppendSeg& g = *segs[i];
      // TQ3 units are 32-token sub-tiles; with a device rollback pending the
      // start's alignment is unknown here, so the span's worst case is taken
      // (the kernel skips a unit left empty)
      const int64_t u = !tq3 ? g.n
                        : c->pend[g.seq] > 0 ? (int64_t)((g.n + 30) / 32 + 1)
                                             : (int64_t)((g.pos0 + g.n - 1) / 32 - g.pos0 / 32 + 1);
      if (units + u > (int64_t)INT32_MAX / 2 && a.n_segs > 0) break;
      a.unit0[a.n_segs] = (int32_t)units;
      a.seq[a.n_segs] = g.seq;
      a.pos0[a.n_segs] = g.pos0;
      a.n[a.n_segs] = g.n;
      a.row0[a.n_segs] = g.src_row0;
      a.keep[a.n_segs] = g.keep_first * kBlock;
      units += u;
      ++a.n_segs;
      ++i;
    }
    a.unit0[a.n_segs] = (int32_t)units;
    a.total_units = (int32_t)units;
    a.roll = c->any_pend ? c->droll : nullptr;
    if (tq3) {
      const Codec& cd = c->core.codec();
      a.signs = c->dsigns;
      a.s_t = c->ds_t;
      for (int j = 0; j < 7; ++j) a.thr[j] = cd.thresholds[j];
      for (int j = 0; j < 8; ++j) a.lev16[j] = cd.levels16[j];
      a.status = c->dstatus;
    }
    const bool with_q = tq3 && qp && i == segs.size();
    hipError_t e = with_q ? launch_append_qprep(a, *qp, s) : launch_append(a, s);
    if (e != hipSuccess) return hip_fail(c, e, "append launch");
    if (with_q && qp_done) *qp_done = true;
  }
  return KV_OK;
}

}  // namespace

extern "C" {

int kv_append(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new, const void* k,
              const void* v, void* stream) {
  if (!c) return KV_EINVAL;
  int rc = check_device(c);
  if (rc != KV_OK) return rc;
  AppendPlan plan;
  std::vector<int32_t> slack = pending_slack(c, n_seqs, seq_ids);
  rc = c->core.plan_append(n_seqs, seq_ids, n_new, &plan, &c->err, slack.data());
  if (rc != KV_OK) return rc;
  if (plan.total_rows > 0 && (!k || !v)) return set_err(c, KV_EINVAL, "null k / v");
  if (plan.total_rows > (int64_t)INT32_MAX / 8) return set_err(c, KV_EINVAL, "append too large");
  rc = enqueue_append(c, plan, slack, k, v, static_cast<hipStream_t>(stream));
  if (rc != KV_OK) return rc;
  c->core.commit_append(plan);
  return KV_OK;
}

int kv_rollback(kv_cache* c, int32_t seq_id, int32_t n_tokens) {
  if (!c) return KV_EINVAL;
  int rc = sync_pending(c);
  if (rc != KV_OK) return rc;
  return c->core.rollback(seq_id, n_tokens, &c->err);
}

int kv_rollback_batch(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_tokens) {
  if (!c) return KV_EINVAL;
  if (n_seqs < 0 || (n_seqs > 0 && (!seq_ids || !n_tokens))) return set_err(c, KV_EINVAL, "bad arrays");
  int rc = sync_pending(c);
  if (rc != KV_OK) return rc;
  std::vector<char> seen(c->core.params().max_seqs, 0);
  for (int i = 0; i < n_seqs; ++i) {
    const int32_t s = seq_ids[i];
    if (!c->core.valid_seq(s)) return set_err(c, KV_ENOSEQ, "sequence id out of range");
    if (seen[s]) return set_err(c, KV_EINVAL, "sequence id repeated");
    seen[s] = 1;
    if (n_tokens[i] < 0) return set_err(c, KV_EINVAL, "rollback count < 0");
    int32_t len;
    c->core.seq_len(s, &len);
    if (n_tokens[i] > len) return set_err(c, KV_ERANGE, "rollback beyond seq_len");
    if (!c->core.window_intact(s, (int64_t)len - n_tokens[i]))
      return set_err(c, KV_ERANGE, "rollback would reach positions a ring cache released");
  }
  for (int i = 0; i < n_seqs; ++i) c->core.rollback(seq_ids[i], n_tokens[i], &c->err);
  return KV_OK;
}

int kv_trace_events(kv_cache* c, void* before, void* after) {
  if (!c) return KV_EINVAL;
  if ((before == nullptr) != (after == nullptr)) return set_err(c, KV_EINVAL, "set both events or neither");
  c->trace_before = static_cast<hipEvent_t>(before);
  c->trace_after = static_cast<hipEvent_t>(after);
  return KV_OK;
}

int kv_seq_free(kv_cache* c, int32_t seq_id) {
  if (!c) return KV_EINVAL;
  int rc = sync_pending(c);
  if (rc != KV_OK) return rc;
  return c->core.free_seq(seq_id, &c->err);
}

int kv_encode(const kv_cache* cc, int64_t n_vecs, const float* src, int32_t is_key, void* dst, void* stream) {
  kv_cache* c = const_cast<kv_cache*>(cc);
  if (!c) return KV_EINVAL;
  if (c->core.params().format != KV_TQ3) return set_err(c, KV_EINVAL, "kv_encode needs a KV_TQ3 handle");
  if (n_vecs < 0) return set_err(c, KV_EINVAL, "n_vecs < 0");
  if (n_vecs > 0 && (!src || !dst)) return set_err(c, KV_EINVAL, "null src / dst");
  if (n_vecs > ((int64_t)1 << 33)) return set_err(c, KV_EINVAL, "n_vecs too large");
  int rc = check_device(c);
  if (rc != KV_OK) return rc;
  const Codec& cd = c->core.codec();
  EncodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.src = src;
  a.dst = static_cast<uint8_t*>(dst);
  a.n = n_vecs;
  a.d = c->core.params().head_dim;
  a.is_key = is_key ? 1 : 0;
  a.signs = c->dsigns;
  a.s_t = c->ds_t;
  for (int j = 0; j < 7; ++j) a.thr[j] = cd.thresholds[j];
  for (int j = 0; j < 8; ++j) a.lev16[j] = cd.levels16[j];
  a.status = c->dstatus;
  hipError_t e = launch_encode(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(c, e, "encode launch");
  return KV_OK;
}

int kv_read_status(kv_cache* c, uint32_t* out, int32_t clear, void* stream) {
  if (!c || !out) return KV_EINVAL;
  int rc = check_device(c);
  if (rc != KV_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, c->dstatus, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess && clear) e = launch_fill_zero(reinterpret_cast<int32_t*>(c->dstatus), 1, s);
  if (e != hipSuccess) return hip_fail(c, e, "reading the status word");
  *out = word;
  return KV_OK;
}

size_t kv_stream_probe_sink_bytes(void) { return (size_t)kProbeWorkgroups * 4; }

int kv_stream_probe(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream) {
  if (!src || !sink || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 ||
      sink_bytes < kv_stream_probe_sink_bytes() || bytes > ((size_t)1 << 40))
    return KV_EINVAL;
  hipError_t e = launch_stream_probe(src, (int64_t)bytes, static_cast<uint32_t*>(sink),
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KV_OK : KV_EDEVICE;
}

}  // extern "C"

namespace {

std::vector<int32_t> pending_slack(const kv_cache* c, int32_t n_seqs, const int32_t* seq_ids) {
  std::vector<int32_t> out(std::max(1, n_seqs), 0);
  for (int i = 0; i < n_seqs && seq_ids; ++i)
    if (c->core.valid_seq(seq_ids[i])) out[i] = c->pend[seq_ids[i]];
  return out;
}

// Read the device rollbacks back and apply them to the host state; blocks
// until the stream of the last kv_rollback_device call gets here.
int sync_pending(kv_cache* c) {
  if (!c->any_pend) return KV_OK;
  const int32_t ms = c->core.params().max_seqs;
  hipError_t e = hipMemcpyAsync(c->h_roll.data(), c->droll, (size_t)ms * 4, hipMemcpyDeviceToHost, c->pend_stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->pend_stream);
  if (e != hipSuccess) return hip_fail(c, e, "reading device rollbacks");
  for (int s = 0; s < ms; ++s)
    if (c->h_roll[s] < 0 || c->h_roll[s] > c->pend[s]) return set_err(c, KV_EDEVICE, "device rollback count out of range");
  for (int s = 0; s < ms; ++s)  // cannot fail: every count was bounded when it was enqueued
    if (c->h_roll[s] > 0 && c->core.rollback(s, c->h_roll[s], &c->err) != KV_OK)
      return set_err(c, KV_EDEVICE, "device rollback past what the host allowed");
  e = launch_fill_zero(c->droll, ms, c->pend_stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->pend_stream);
  if (e != hipSuccess) return hip_fail(c, e, "clearing device rollbacks");
  std::fill(c->pend.begin(), c->pend.end(), 0);
  c->any_pend = false;
  return KV_OK;
}

// Checks of a verify call beyond its plan.
int check_verify_args(kv_cache* c, const VerifyPlan& vp, const float* q, float scale, float softcap, float* out,
                      void* workspace, size_t ws_bytes) {
  if (!q || !out) return set_err(c, KV_EINVAL, "null q / out");
  if (!std::isfinite(scale)) return set_err(c, KV_EINVAL, "scale must be finite");
  if (!(softcap >= 0.0f) || !std::isfinite(softcap)) return set_err(c, KV_EINVAL, "softcap must be finite and >= 0");
  if (ws_bytes < vp.total) return set_err(c, KV_ENOMEM, "workspace too small");
  if (vp.total > 0 && (!workspace || reinterpret_cast<uintptr_t>(workspace) % kAlign))
    return set_err(c, KV_EINVAL, "workspace must be non-null and 256-byte aligned");
  return KV_OK;
}

// Enqueue table updates for the blocks an append plan pops.
int enqueue_table_updates(kv_cache* c, const AppendPlan& plan, hipStream_t s) {
  for (size_t i = 0; i < plan.popped.size(); i += kMaxTableUpdates) {
    TableUpdateArgs ta;
    ta.table = c->dtable;
    ta.count = (int32_t)std::min<size_t>(kMaxTableUpdates, plan.popped.size() - i);
    for (int j = 0; j < ta.count; ++j) {
      ta.index[j] = plan.table_index[i + j];
      ta.block[j] = plan.popped[i + j];
    }
    hipError_t e = launch_table_update(ta, s);
    if (e != hipSuccess) return hip_fail(c, e, "table update launch");
  }
  return KV_OK;
}

// TQ3: the rotation of a verify call's queries; q' = Pi q and q'' = S q'
// live in the workspace after the partials.
QPrepArgs make_qprep(const kv_cache* c, const VerifyPlan& vp, const float* q, int32_t num_q_heads, void* workspace) {
  QPrepArgs qa;
  qa.q = q;
  qa.q1 = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + vp.part_bytes);
  qa.q2 = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + vp.part_bytes + vp.q_bytes);
  qa.signs = c->dsigns;
  qa.s_t = c->ds_t;
  qa.n_vec = (int32_t)(vp.rows * num_q_heads);
  qa.d = c->core.params().head_dim;
  return qa;
}

// Enqueue a planned verify call.  added / new_k / new_v: a fused append of
// the verified rows (plain formats; the table already holds their blocks),
// else null.  rotated: TQ3 queries already rotated into the workspace.
int enqueue_verify(kv_cache* c, const VerifyPlan& vp, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows,
                   const int32_t* added, const float* q, int32_t num_q_heads, float scale, float softcap,
                   int32_t window, float* out, void* workspace, hipStream_t s, const void* new_k, const void* new_v,
                   bool rotated = false, bool valu = false) {
  const CoreParams& P = c->core.params();
  const bool tq3 = P.format == KV_TQ3;
  float* q1 = nullptr;
  float* q2 = nullptr;
  if (tq3) {
    const QPrepArgs qa = make_qprep(c, vp, q, num_q_heads, workspace);
    q1 = qa.q1;
    q2 = qa.q2;
    if (!rotated) {
      hipError_t e = launch_qprep(qa, s);
      if (e != hipSuccess) return hip_fail(c, e, "query rotation launch");
    }
  }
  const int g = num_q_heads / P.num_kv_heads;
  // one set of launches per head slice, each over its own block of partial
  // slots; the fused append rides on the first slice only (the later
  // slices' launches follow it on the stream and read the rows it stored)
  const size_t nl = vp.launches.size();
  std::vector<AttnArgs> args(vp.hs * nl);
  std::vector<char> split(args.size(), 0);
  for (size_t ai = 0; ai < args.size(); ++ai) {
    const int slice = (int)(ai / nl);
    const VerifyLaunch& L = vp.launches[ai % nl];
    AttnArgs& a = args[ai];
    std::memset(&a, 0, sizeof(a));
    a.pool = c->pool;
    a.table = c->dtable;
    a.signs = c->dsigns;
    a.q = tq3 ? q1 : q;
    a.q2 = q2;
    a.inv_sqrt_d = 1.0f / std::sqrt((float)P.head_dim);
    a.qjl_coef = (float)(std::sqrt(M_PI / 2.0) / P.head_dim);
    a.q1_mul = (float)((double)scale * M_LOG2E / std::sqrt((double)P.head_dim));
    a.q2_mul = (float)(std::sqrt(M_PI / 2.0) / std::sqrt((double)P.head_dim));
    a.cap_l2 = (float)((double)softcap * M_LOG2E);
    a.inv_cap_l2 = softcap > 0.0f ? (float)(1.0 / ((double)softcap * M_LOG2E)) : 0.0f;
    for (int j = 0; j < 8; ++j) a.lev16_bits[j] = tq3 ? c->core.codec().levels16_bits[j] : 0;
    a.out = out;
    a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace)) + (slice * vp.slots + L.slot0) * vp.slot_stride;
    a.lay = c->lay;
    a.hq = num_q_heads;
    a.g = vp.gs;
    a.gq = g;
    a.head0 = slice * vp.gs;
    a.max_bps = P.max_blocks_per_seq;
    a.window = window;
    a.scale = scale;
    a.softcap = softcap;
    a.inv_softcap = softcap > 0.0f ? 1.0f / softcap : 0.0f;
    a.n_seqs = L.count;
    a.n_wg = L.n_wg;
    a.slot_stride = (int32_t)vp.slot_stride;
    a.rpad = vp.rpad;
    a.force_partial = tq3 ? 1 : 0;  // the merge rotates TQ3 outputs back
    a.tile_keys = tile_keys(P.format, P.head_dim);
    a.roll = c->any_pend ? c->droll : nullptr;
    a.new_k = slice == 0 ? new_k : nullptr;
    a.new_v = slice == 0 ? new_v : nullptr;
    bool any_split = tq3;
    for (int i = 0; i < L.count; ++i) {
      const int ci = vp.order[L.first + i];
      const int sid = seq_ids[ci];
      int32_t up, low;
      verify_lengths(c, sid, added ? added[ci] : 0, &up, &low);
      a.seq[i] = sid;
      a.len[i] = up;
      a.qrow0[i] = vp.qrow0[ci];
      a.nrows[i] = n_rows[ci];
      a.ksplit[i] = L.ksplit[i];
      if (L.ksplit[i] > 1) any_split = true;
    }
    for (int i = 0; i <= L.count; ++i) a.wg_base[i] = L.wg_base[i];
    split[ai] = any_split ? 1 : 0;
  }
  hipError_t e = hipSuccess;
  if (c->trace_before) e = hipEventRecord(c->trace_before, s);
  for (size_t li = 0; li < args.size() && e == hipSuccess; ++li)
    e = valu  ? launch_attn_valu(args[li], s)
        : tq3 ? launch_attn_tq3(args[li], vp.nct, s)
              : launch_attn(args[li], vp.nct, s);
  if (e == hipSuccess && c->trace_after) e = hipEventRecord(c->trace_after, s);
  if (e != hipSuccess) return hip_fail(c, e, "attention launch");
  for (size_t li = 0; li < args.size(); ++li) {
    if (!split[li]) continue;
    e = launch_merge(args[li], vp.nct, s);
    if (e != hipSuccess) return hip_fail(c, e, "merge launch");
  }
  return KV_OK;
}

}  // namespace

extern "C" {

int kv_workspace_bytes(const kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows,
                       int32_t num_q_heads, int32_t window, size_t* out) {
  if (!c || !out) return KV_EINVAL;
  VerifyPlan vp;
  int rc = plan_verify(c, n_seqs, seq_ids, n_rows, num_q_heads, window, nullptr, &vp,
                       &const_cast<kv_cache*>(c)->err);
  if (rc != KV_OK) return rc;
  *out = vp.total;
  return KV_OK;
}

int kv_append_verify_workspace_bytes(const kv_cache* c, int32_t n_seqs, const int32_t* seq_ids,
                                     const int32_t* n_rows, int32_t num_q_heads, int32_t window, size_t* out) {
  if (!c || !out) return KV_EINVAL;
  VerifyPlan vp;
  int rc = plan_verify(c, n_seqs, seq_ids, n_rows, num_q_heads, window, n_rows, &vp,
                       &const_cast<kv_cache*>(c)->err);
  if (rc != KV_OK) return rc;
  *out = vp.total;
  return KV_OK;
}

int spec_verify_attn(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows, const float* q,
                     int32_t num_q_heads, float scale, float softcap, int32_t window, float* out, void* workspace,
                     size_t ws_bytes, void* stream) {
  if (!c) return KV_EINVAL;
  int rc = check_device(c);
  if (rc != KV_OK) return rc;
  VerifyPlan vp;
  rc = plan_verify(c, n_seqs, seq_ids, n_rows, num_q_heads, window, nullptr, &vp, &c->err);
  if (rc != KV_OK) return rc;
  rc = check_verify_args(c, vp, q, scale, softcap, out, workspace, ws_bytes);
  if (rc != KV_OK) return rc;
  return enqueue_verify(c, vp, n_seqs, seq_ids, n_rows, nullptr, q, num_q_heads, scale, softcap, window, out,
                        workspace, static_cast<hipStream_t>(stream), nullptr, nullptr);
}

int kv_workspace_bytes_valu(const kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows,
                            int32_t num_q_heads, int32_t window, size_t* out) {
  if (!c || !out) return KV_EINVAL;
  VerifyPlan vp;
  int rc = plan_verify_valu(c, n_seqs, seq_ids, n_rows, num_q_heads, window, &vp);
  if (rc != KV_OK) return rc;
  *out = vp.total;
  return KV_OK;
}

int spec_verify_attn_valu(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows, const float* q,
                          int32_t num_q_heads, float scale, float softcap, int32_t window, float* out,
                          void* workspace, size_t ws_bytes, void* stream) {
  if (!c) return KV_EINVAL;
  int rc = check_device(c);
  if (rc != KV_OK) return rc;
  VerifyPlan vp;
  rc = plan_verify_valu(c, n_seqs, seq_ids, n_rows, num_q_heads, window, &vp);
  if (rc != KV_OK) return rc;
  rc = check_verify_args(c, vp, q, scale, softcap, out, workspace, ws_bytes);
  if (rc != KV_OK) return rc;
  return enqueue_verify(c, vp, n_seqs, seq_ids, n_rows, nullptr, q, num_q_heads, scale, softcap, window, out,
                        workspace, static_cast<hipStream_t>(stream), nullptr, nullptr, false, true);
}

int spec_verify_attn_static(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows,
                            const float* q, int32_t num_q_heads, float scale, float softcap, int32_t window,
                            float* out, void* stream) {
  if (!c) return KV_EINVAL;
  int rc = check_device(c);
  if (rc != KV_OK) return rc;
  VerifyPlan vp;
  rc = plan_verify(c, n_seqs, seq_ids, n_rows, num_q_heads, window, nullptr, &vp, &c->err);
  if (rc != KV_OK) return rc;
  if (vp.total > kStaticScratchBytes)
    return set_err(c, KV_ENOMEM,
                   "call needs " + std::to_string(vp.total) + " bytes of scratch; the fixed scratch holds " +
                       std::to_string(kStaticScratchBytes) + " (use spec_verify_attn with a workspace)");
  void* ws = nullptr;
  hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return hip_fail(c, e, "resolving the fixed scratch");
  rc = check_verify_args(c, vp, q, scale, softcap, out, ws, kStaticScratchBytes);
  if (rc != KV_OK) return rc;
  return enqueue_verify(c, vp, n_seqs, seq_ids, n_rows, nullptr, q, num_q_heads, scale, softcap, window, out, ws,
                        static_cast<hipStream_t>(stream), nullptr, nullptr);
}

int kv_append_verify(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_rows, const void* k,
                     const void* v, const float* q, int32_t num_q_heads, float scale, float softcap, int32_t window,
                     float* out, void* workspace, size_t ws_bytes, void* stream) {
  if (!c) return KV_EINVAL;
  int rc = check_device(c);
  if (rc != KV_OK) return rc;
  AppendPlan plan;
  std::vector<int32_t> slack = pending_slack(c, n_seqs, seq_ids);
  rc = c->core.plan_append(n_seqs, seq_ids, n_rows, &plan, &c->err, slack.data());
  if (rc != KV_OK) return rc;
  VerifyPlan vp;
  rc = plan_verify(c, n_seqs, seq_ids, n_rows, num_q_heads, window, n_rows, &vp, &c->err);
  if (rc != KV_OK) return rc;
  rc = check_verify_args(c, vp, q, scale, softcap, out, workspace, ws_bytes);
  if (rc != KV_OK) return rc;
  if (!k || !v) return set_err(c, KV_EINVAL, "null k / v");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const CoreParams& P = c->core.params();
  // Plain formats: the attention kernel writes the rows (no launch of its
  // own; a table update goes first when blocks are popped, about once per
  // 256 / rows steps of a sequence).  TQ3 encodes in its own launch.
  const bool fused = P.format != KV_TQ3 && reinterpret_cast<uintptr_t>(k) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(v) % 16 == 0;  // the kernel reads rows in 16-byte pieces
  if (!fused) {
    // the append's launches, then the verify planned with the appended
    // lengths; the host state moves only once both are enqueued
    if (plan.total_rows > (int64_t)INT32_MAX / 8) return set_err(c, KV_EINVAL, "append too large");
    // TQ3: the queries are rotated in the append's (last) launch, beside the
    // encode
    const QPrepArgs qa = make_qprep(c, vp, q, num_q_heads, workspace);
    bool rotated = false;
    rc = enqueue_append(c, plan, slack, k, v, s, P.format == KV_TQ3 ? &qa : nullptr, &rotated);
    if (rc != KV_OK) return rc;
    rc = enqueue_verify(c, vp, n_seqs, seq_ids, n_rows, n_rows, q, num_q_heads, scale, softcap, window, out,
                        workspace, s, nullptr, nullptr, rotated);
    if (rc != KV_OK) return rc;
    c->core.commit_append(plan);
    return KV_OK;
  }
  rc = enqueue_table_updates(c, plan, s);
  if (rc != KV_OK) return rc;
  rc = enqueue_verify(c, vp, n_seqs, seq_ids, n_rows, n_rows, q, num_q_heads, scale, softcap, window, out, workspace,
                      s, k, v);
  if (rc != KV_OK) return rc;
  c->core.commit_append(plan);
  return KV_OK;
}

int kv_rollback_device(kv_cache* c, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_draft,
                       const int32_t* accepted, void* stream) {
  if (!c) return KV_EINVAL;
  int rc = check_device(c);
  if (rc != KV_OK) return rc;
  if (n_seqs < 0 || (n_seqs > 0 && (!seq_ids || !n_draft || !accepted)))
    return set_err(c, KV_EINVAL, "bad arrays");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (c->any_pend && s != c->pend_stream)
    return set_err(c, KV_EINVAL, "pending device rollbacks were enqueued on another stream; call kv_sync first");
  std::vector<char> seen(c->core.params().max_seqs, 0);
  for (int i = 0; i < n_seqs; ++i) {
    const int32_t sid = seq_ids[i];
    if (!c->core.valid_seq(sid)) return set_err(c, KV_ENOSEQ, "sequence id out of range");
    if (seen[sid]) return set_err(c, KV_EINVAL, "sequence id repeated");
    seen[sid] = 1;
    if (n_draft[i] < 0) return set_err(c, KV_EINVAL, "n_draft < 0");
    int32_t up, low;
    verify_lengths(c, sid, 0, &up, &low);
    if (n_draft[i] > low) return set_err(c, KV_ERANGE, "n_draft exceeds the sequence's length");
    if (!c->core.window_intact(sid, (int64_t)low - n_draft[i]))
      return set_err(c, KV_ERANGE, "rollback could reach positions a ring cache released");
  }
  for (int first = 0; first < n_seqs; first += kMaxRollback) {
    RollbackArgs a;
    std::memset(&a, 0, sizeof(a));
    a.roll = c->droll;
    a.accepted = accepted + first;
    a.count = std::min(kMaxRollback, n_seqs - first);
    for (int i = 0; i < a.count; ++i) {
      a.seq[i] = seq_ids[first + i];
      a.n_draft[i] = n_draft[first + i];
    }
    hipError_t e = launch_rollback(a, s);
    if (e != hipSuccess) return hip_fail(c, e, "rollback launch");
  }
  for (int i = 0; i < n_seqs; ++i) {
    if (n_draft[i] == 0) continue;
    c->pend[seq_ids[i]] += n_draft[i];
    c->any_pend = true;
    c->pend_stream = s;
  }
  return KV_OK;
}

int kv_sync(kv_cache* c) {
  if (!c) return KV_EINVAL;
  return sync_pending(c);
}

int kv_seq_len(const kv_cache* c, int32_t seq_id, int32_t* out) {
  if (!c || !out) return KV_EINVAL;
  int rc = sync_pending(const_cast<kv_cache*>(c));
  if (rc != KV_OK) return rc;
  return c->core.seq_len(seq_id, out);
}

int kv_block_table(const kv_cache* c, int32_t seq_id, int32_t* out, int32_t cap, int32_t* n_owned) {
  if (!c || !n_owned || cap < 0 || (cap > 0 && !out)) return KV_EINVAL;
  int rc = sync_pending(const_cast<kv_cache*>(c));
  if (rc != KV_OK) return rc;
  int32_t owned;
  rc = c->core.owned(seq_id, &owned);
  if (rc != KV_OK) return rc;
  const int32_t* row = c->core.table_row(seq_id);
  for (int i = 0; i < std::min(cap, owned); ++i) out[i] = row[i];
  *n_owned = owned;
  return KV_OK;
}

int kv_free_blocks(const kv_cache* c, int32_t* out) {
  if (!c || !out) return KV_EINVAL;
  *out = c->core.free_count();
  return KV_OK;
}

int kv_codec(const kv_cache* c, int8_t* signs, float* s_matrix, double* levels, double* levels16,
             double* thresholds) {
  if (!c) return KV_EINVAL;
  if (c->core.params().format != KV_TQ3) return KV_EINVAL;
  const Codec& cd = c->core.codec();
  const int d = cd.d;
  if (signs) std::memcpy(signs, cd.signs.data(), d);
  if (s_matrix) std::memcpy(s_matrix, cd.s.data(), (size_t)d * d * 4);
  if (levels) std::memcpy(levels, cd.levels, sizeof(cd.levels));
  if (levels16) std::memcpy(levels16, cd.levels16, sizeof(cd.levels16));
  if (thresholds) std::memcpy(thresholds, cd.thresholds, sizeof(cd.thresholds));
  return KV_OK;
}

const char* kv_last_error(const kv_cache* c) { return c ? c->err.c_str() : "null handle"; }

}  // extern "C"

// ---- acceptance of drafts ---------------------------------------------------------

namespace {

thread_local std::string g_accept_err;

int accept_fail(int code, const char* msg) {
  g_accept_err = msg;
  return code;
}

struct AcceptLayout {
  int64_t rows_t = 0, rows_d = 0, nch = 0;
  size_t stats_off = 0, plan_off = 0, fsum_off = 0, total = 0;
};

int accept_layout(int32_t n_seqs, const int32_t* n_draft, int32_t vocab, bool with_draft, float temperature,
                  AcceptLayout* L) {
  if (n_seqs < 0) return accept_fail(KV_EINVAL, "n_seqs must be >= 0");
  if (n_seqs > 0 && !n_draft) return accept_fail(KV_EINVAL, "null n_draft");
  if (vocab < 1) return accept_fail(KV_EINVAL, "vocab must be >= 1");
  if (!std::isfinite(temperature) || temperature < 0.0f)
    return accept_fail(KV_EINVAL, "temperature must be finite and >= 0");
  int64_t nd = 0;
  for (int i = 0; i < n_seqs; ++i) {
    if (n_draft[i] < 0 || n_draft[i] > KV_MAX_ROWS - 1) return accept_fail(KV_EINVAL, "n_draft must be in [0, 7]");
    nd += n_draft[i];
  }
  L->rows_t = nd + n_seqs;
  L->rows_d = (with_draft && temperature > 0.0f) ? nd : 0;
  L->nch = (vocab + kAcceptChunk - 1) / kAcceptChunk;
  L->stats_off = 0;
  L->plan_off = align_up((size_t)(L->rows_t + L->rows_d) * L->nch * 16);
  L->fsum_off = L->plan_off + align_up((size_t)n_seqs * sizeof(AcceptPlan));
  L->total = L->fsum_off + align_up((size_t)n_seqs * L->nch * 4);
  return KV_OK;
}

}  // namespace

extern "C" {

int spec_accept_workspace_bytes(int32_t n_seqs, const int32_t* n_draft, int32_t vocab, int32_t with_draft,
                                float temperature, size_t* out) {
  if (!out) return accept_fail(KV_EINVAL, "null out");
  AcceptLayout L;
  const int rc = accept_layout(n_seqs, n_draft, vocab, with_draft != 0, temperature, &L);
  if (rc != KV_OK) return rc;
  *out = L.total;
  return KV_OK;
}

int spec_accept(int32_t n_seqs, const int32_t* n_draft, int32_t vocab, const float* target_logits,
                const float* draft_logits, const int32_t* draft_tokens, const float* uniforms, float temperature,
                int32_t* out_accepted, int32_t* out_token, void* workspace, size_t ws_bytes, void* stream) {
  AcceptLayout L;
  int rc = accept_layout(n_seqs, n_draft, vocab, draft_logits != nullptr, temperature, &L);
  if (rc != KV_OK) return rc;
  if (n_seqs == 0) return KV_OK;
  if (!target_logits || !uniforms || !out_accepted || !out_token)
    return accept_fail(KV_EINVAL, "null target_logits / uniforms / outputs");
  if (L.rows_t > n_seqs && !draft_tokens) return accept_fail(KV_EINVAL, "null draft_tokens");
  if (ws_bytes < L.total) return accept_fail(KV_ENOMEM, "workspace too small");
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return accept_fail(KV_EINVAL, "workspace must be non-null and 256-byte aligned");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return accept_fail(KV_EDEVICE, hipGetErrorString(e));
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  AcceptArgs a;
  std::memset(&a, 0, sizeof(a));
  a.target = target_logits;
  a.draft = L.rows_d > 0 ? draft_logits : nullptr;
  a.drafts = draft_tokens;
  a.u = uniforms;
  a.out_acc = out_accepted;
  a.out_tok = out_token;
  a.stats = reinterpret_cast<float4*>(ws + L.stats_off);
  a.plan = reinterpret_cast<AcceptPlan*>(ws + L.plan_off);
  a.fsum = reinterpret_cast<float*>(ws + L.fsum_off);
  a.inv_t = temperature > 0.0f ? 1.0f / temperature : 0.0f;
  a.vocab = vocab;
  a.nch = (int32_t)L.nch;
  a.rows_t = (int32_t)L.rows_t;
  a.rows_d = (int32_t)L.rows_d;
  e = launch_accept_stats(a, s);
  if (e != hipSuccess) return accept_fail(KV_EDEVICE, hipGetErrorString(e));
  int32_t t0 = 0, d0 = 0;
  for (int first = 0; first < n_seqs; first += kMaxAcceptSeqs) {
    a.seq0 = first;
    a.count = std::min(kMaxAcceptSeqs, n_seqs - first);
    for (int i = 0; i < a.count; ++i) {
      a.n[i] = n_draft[first + i];
      a.t0[i] = t0;
      a.d0[i] = d0;
      t0 += n_draft[first + i] + 1;
      d0 += n_draft[first + i];
    }
    e = launch_accept_group(a, s);
    if (e != hipSuccess) return accept_fail(KV_EDEVICE, hipGetErrorString(e));
  }
  return KV_OK;
}

const char* spec_accept_last_error(void) { return g_accept_err.c_str(); }

}  // extern "C"
