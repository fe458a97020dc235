// plan.cpp - host planning of a verify call (see plan.h), HIP-free: linked
// into libsvattn.so and into the host-only core library.
#include "plan.h"

#include <algorithm>
#include <cstdio>
#include <cstdlib>

#include "svattn.h"

namespace svattn {

void verify_lengths(const Core& core, const int32_t* pend, int32_t seq, int32_t added, int32_t* up, int32_t* low) {
  int32_t len = 0;
  core.seq_len(seq, &len);
  *up = len + added;
  *low = *up - (pend ? pend[seq] : 0);
}

int plan_verify(const Core& core, const int32_t* pend, int32_t n_seqs, const int32_t* seq_ids,
                const int32_t* n_rows, int32_t num_q_heads, int32_t window, const int32_t* added, VerifyPlan* vp,
                std::string* err, int max_cols) {
  *vp = VerifyPlan();
  const CoreParams& P = core.params();
  auto fail = [&](int code, const std::string& m) {
    if (err) *err = m;
    return code;
  };
  if (n_seqs < 1) return fail(KV_EINVAL, "n_seqs must be >= 1");
  if (!seq_ids || !n_rows) return fail(KV_EINVAL, "null seq_ids / n_rows");
  if (num_q_heads < 1 || num_q_heads % P.num_kv_heads) return fail(KV_EINVAL, "num_q_heads must be a multiple of num_kv_heads");
  if (window < 0) return fail(KV_EINVAL, "window < 0");
  if (P.ring_window > 0 && (window < 1 || window > P.ring_window))
    return fail(KV_EINVAL, "a ring cache serves windows of 1 .. " + std::to_string(P.ring_window) + " positions");
  const int g = num_q_heads / P.num_kv_heads;
  int max_rows = 0;
  for (int i = 0; i < n_seqs; ++i) {
    if (!core.valid_seq(seq_ids[i])) return fail(KV_ENOSEQ, "sequence id " + std::to_string(seq_ids[i]) + " out of range");
    int32_t up, low;
    verify_lengths(core, pend, seq_ids[i], added ? added[i] : 0, &up, &low);
    if (n_rows[i] < 1 || n_rows[i] > KV_MAX_ROWS) return fail(KV_EINVAL, "n_rows must be in [1, 8]");
    if (n_rows[i] > low)
      return fail(KV_ERANGE, "n_rows exceeds seq_len of sequence " + std::to_string(seq_ids[i]) +
                                 (up > low ? " (device rollbacks pending: the lower bound counts)" : ""));
    if (P.ring_window > 0 && std::max(0, low - n_rows[i] - window + 1) < core.first_block(seq_ids[i]) * kBlock)
      return fail(KV_ERANGE, "the rows' windows reach positions the ring cache released");
    max_rows = std::max(max_rows, (int)n_rows[i]);
    vp->rows += n_rows[i];
  }
  // head slices: the fewest that bring a slice's columns to max_cols or
  // fewer (hs = g always works: one head per slice, at most 8 rows)
  if (max_cols == 0) max_cols = mfma_max_cols(P.format, P.head_dim);
  if (max_cols < 8 || max_cols > 64) return fail(KV_EINVAL, "column cap");
  vp->hs = 1;
  while (g % vp->hs || max_rows * (g / vp->hs) > max_cols) ++vp->hs;
  vp->gs = g / vp->hs;
  const int R = max_rows * vp->gs;
  vp->nct = R > 32 ? 2 : 1;
  vp->rpad = 32 * vp->nct;
  vp->slot_stride = (int64_t)vp->rpad * (2 + P.head_dim);
  const int TL = 4 / vp->nct;
  const int target_wg = P.head_dim > 128 ? SVATTN_WG_PER_CALL_D256 : SVATTN_WG_PER_CALL;
  // tiles of each (sequence, kv head) pair over the whole call
  const int tk = tile_keys(P.format, P.head_dim);
  std::vector<int> nt(n_seqs);
  int64_t total_tiles = 0;
  for (int i = 0; i < n_seqs; ++i) {
    int32_t up, low;
    verify_lengths(core, pend, seq_ids[i], added ? added[i] : 0, &up, &low);
    const int klo = window > 0 ? std::max(0, low - n_rows[i] - window + 1) : 0;
    nt[i] = (up + tk - 1) / tk - klo / tk;
    total_tiles += (int64_t)nt[i] * P.num_kv_heads;
  }
  // Uniform batches: one round of workgroups (one per CU).  Ragged batches
  // (lengths far apart): four times as many, smaller chunks, so the dispatcher
  // can even out the mix of long and short pairs.
  const int nt_max = *std::max_element(nt.begin(), nt.end());
  const int nt_min = *std::min_element(nt.begin(), nt.end());
  const int64_t target = 4 * (int64_t)nt_min >= 3 * (int64_t)nt_max ? target_wg : 4 * (int64_t)target_wg;
  // chunks of at most ~total / target tiles, never fewer than one per token lane
  const int64_t per_wg = std::max<int64_t>(TL, (total_tiles + target - 1) / target);
  // Sequences go to the kernel longest first (workgroups are dispatched in
  // index order, so the big chunks start first and the short ones fill in).
  vp->order.resize(n_seqs);
  for (int i = 0; i < n_seqs; ++i) vp->order[i] = i;
  std::stable_sort(vp->order.begin(), vp->order.end(), [&](int x, int y) { return nt[x] > nt[y]; });
  vp->qrow0.assign(n_seqs, 0);
  for (int i = 1; i < n_seqs; ++i) vp->qrow0[i] = vp->qrow0[i - 1] + n_rows[i - 1];
  for (int first = 0; first < n_seqs; first += kMaxAttnSeqs) {
    VerifyLaunch L;
    L.first = first;
    L.count = std::min(kMaxAttnSeqs, n_seqs - first);
    L.ksplit.assign(L.count, 1);
    L.wg_base.assign(L.count + 1, 0);
    for (int i = 0; i < L.count; ++i) {
      const int tiles = nt[vp->order[first + i]];
      int k = (int)std::max<int64_t>(1, (tiles + per_wg - 1) / per_wg);
      const int cs = (tiles + k - 1) / k;
      k = (tiles + cs - 1) / cs;  // no empty chunk
      L.ksplit[i] = k;
      L.wg_base[i + 1] = L.wg_base[i] + k * P.num_kv_heads;
    }
    L.n_wg = L.wg_base[L.count];
    L.slot0 = vp->slots;
    vp->slots += L.n_wg;
    vp->launches.push_back(std::move(L));
  }
  vp->part_bytes = align_up((size_t)vp->hs * vp->slots * vp->slot_stride * 4);
  if (P.format == KV_TQ3) vp->q_bytes = align_up((size_t)vp->rows * num_q_heads * P.head_dim * 4);
  vp->total = vp->part_bytes + 2 * vp->q_bytes;
#ifdef SVATTN_CHECKED
  const std::string bad = check_plan(core, pend, n_seqs, seq_ids, n_rows, num_q_heads, window, added, *vp, max_cols);
  if (!bad.empty()) {
    std::fprintf(stderr, "svattn: verify plan violates its invariants: %s\n", bad.c_str());
    std::abort();
  }
#endif
  return KV_OK;
}

std::string check_plan(const Core& core, const int32_t* pend, int32_t n_seqs, const int32_t* seq_ids,
                       const int32_t* n_rows, int32_t num_q_heads, int32_t window, const int32_t* added,
                       const VerifyPlan& vp, int max_cols) {
  const CoreParams& P = core.params();
  auto str = [](int64_t x) { return std::to_string(x); };
  if (max_cols == 0) max_cols = mfma_max_cols(P.format, P.head_dim);
  if (n_seqs < 1) return "no sequences";
  const int g = num_q_heads / P.num_kv_heads;
  // rows and column groups: every query column of a (sequence, kv head) pair
  // fits the plan's column groups
  int max_rows = 0;
  int64_t rows = 0;
  for (int i = 0; i < n_seqs; ++i) {
    max_rows = std::max<int>(max_rows, n_rows[i]);
    rows += n_rows[i];
  }
  if (vp.rows != rows) return "rows " + str(vp.rows) + " != " + str(rows);
  // head slices: hs x gs = g, a slice's columns fit two 32-column groups,
  // and no smaller number of slices would do
  if (vp.hs < 1 || vp.gs < 1 || vp.hs * vp.gs != g) return "head slices " + str(vp.hs) + " x " + str(vp.gs);
  if (max_rows * vp.gs > max_cols) return "slice columns " + str(max_rows * vp.gs);
  for (int h2 = 1; h2 < vp.hs; ++h2)
    if (g % h2 == 0 && max_rows * (g / h2) <= max_cols) return "fewer head slices would do: " + str(h2);
  if (vp.nct != 1 && vp.nct != 2) return "column groups " + str(vp.nct);
  if (vp.rpad != 32 * vp.nct) return "padded columns " + str(vp.rpad);
  if (max_rows * vp.gs > vp.rpad || (vp.nct == 2 && max_rows * vp.gs <= 32))
    return "columns " + str(max_rows * vp.gs) + " vs " + str(vp.rpad);
  if (vp.slot_stride != (int64_t)vp.rpad * (2 + P.head_dim)) return "slot stride";
  // row offsets: prefix sums of the row counts, in call order
  if ((int)vp.qrow0.size() != n_seqs) return "qrow0 size";
  for (int i = 0, r = 0; i < n_seqs; r += n_rows[i], ++i)
    if (vp.qrow0[i] != r) return "qrow0[" + str(i) + "]";
  // kernel order: a permutation of the call, longest pair first
  if ((int)vp.order.size() != n_seqs) return "order size";
  const int tk = tile_keys(P.format, P.head_dim);
  std::vector<int> seen(n_seqs, 0), nt(n_seqs, 0);
  for (int i = 0; i < n_seqs; ++i) {
    int32_t up, low;
    verify_lengths(core, pend, seq_ids[i], added ? added[i] : 0, &up, &low);
    const int klo = window > 0 ? std::max(0, low - n_rows[i] - window + 1) : 0;
    nt[i] = (up + tk - 1) / tk - klo / tk;
    if (nt[i] < 1) return "sequence " + str(i) + " has no tile";
  }
  for (int i = 0; i < n_seqs; ++i) {
    const int ci = vp.order[i];
    if (ci < 0 || ci >= n_seqs || seen[ci]++) return "order is not a permutation at " + str(i);
    if (i > 0 && nt[vp.order[i - 1]] < nt[ci]) return "order not longest first at " + str(i);
  }
  // launches (of one head slice; every slice repeats them with its own
  // block of `slots` partial slots): consecutive runs of at most
  // kMaxAttnSeqs sequences; inside one, sequence i owns workgroups
  // wg_base[i] .. wg_base[i+1]-1, ksplit[i] chunks per kv head, each chunk a
  // non-empty run of tiles, one partial slot per workgroup
  int first = 0;
  int64_t slot = 0;
  for (size_t li = 0; li < vp.launches.size(); ++li) {
    const VerifyLaunch& L = vp.launches[li];
    const std::string at = "launch " + str((int64_t)li) + ": ";
    if (L.first != first || L.count < 1 || L.count > kMaxAttnSeqs || L.first + L.count > n_seqs)
      return at + "sequence range";
    if ((int)L.ksplit.size() != L.count || (int)L.wg_base.size() != L.count + 1) return at + "table sizes";
    if (L.wg_base[0] != 0) return at + "wg_base[0]";
    for (int i = 0; i < L.count; ++i) {
      const int k = L.ksplit[i], t = nt[vp.order[L.first + i]];
      if (k < 1 || k > t) return at + "ksplit[" + str(i) + "] = " + str(k) + " for " + str(t) + " tiles";
      const int cs = (t + k - 1) / k;
      if ((int64_t)(k - 1) * cs >= t) return at + "empty chunk of sequence " + str(i);
      if (L.wg_base[i + 1] - L.wg_base[i] != k * P.num_kv_heads) return at + "wg_base[" + str(i + 1) + "]";
    }
    if (L.n_wg != L.wg_base[L.count] || L.n_wg < 1) return at + "workgroup count";
    if (L.slot0 != slot) return at + "first slot";
    slot += L.n_wg;
    first += L.count;
  }
  if (first != n_seqs) return "launches cover " + str(first) + " of " + str(n_seqs) + " sequences";
  if (vp.slots != slot) return "slots";
  // workspace: partial slots, then (compressed caches) two rotated copies of
  // the queries
  if (vp.part_bytes != align_up((size_t)vp.hs * vp.slots * vp.slot_stride * 4)) return "partial bytes";
  const size_t q = P.format == KV_TQ3 ? align_up((size_t)rows * num_q_heads * P.head_dim * 4) : 0;
  if (vp.q_bytes != q) return "query bytes";
  if (vp.total != vp.part_bytes + 2 * vp.q_bytes) return "total bytes";
  return std::string();
}

}  // namespace svattn
