// ngram.cpp - the n-gram self-drafter behind include/svdraft.h (host only).
//
// AX Engine page, "Core Technical Architecture & Methods": bigram/trigram
// tables built at run time, up to 4 drafts per step, an EMA acceptance gate
// (tau 0.1, threshold 0.5).  The rules this file follows are listed in the
// header.  Each sequence keeps its last two tokens, a position counter and
// two hash maps from context to a short list of (token, count, last seen).
#include <cstdint>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

#include "svdraft.h"

namespace {

constexpr int kEinval = -1, kEnoseq = -4;
constexpr int kMaxDrafts = 7;

struct Cont {
  int32_t token;
  int32_t count;
  int64_t last;  // position of its latest occurrence
};

// Continuations of one context; few per context, so a flat list.
struct Conts {
  std::vector<Cont> v;
  void add(int32_t t, int64_t pos) {
    for (Cont& c : v)
      if (c.token == t) {
        ++c.count;
        c.last = pos;
        return;
      }
    v.push_back(Cont{t, 1, pos});
  }
  int32_t best() const {  // most frequent, then latest
    const Cont* b = &v[0];
    for (const Cont& c : v)
      if (c.count > b->count || (c.count == b->count && c.last > b->last)) b = &c;
    return b->token;
  }
};

struct SeqState {
  int64_t seen = 0;  // tokens observed
  int32_t prev1 = -1, prev2 = -1;
  std::unordered_map<uint64_t, Conts> tri;
  std::unordered_map<int32_t, Conts> bi;
  double rate = 1.0;
  std::vector<int32_t> pending;
};

uint64_t pair_key(int32_t a, int32_t b) { return ((uint64_t)(uint32_t)a << 32) | (uint32_t)b; }

}  // namespace

struct ngram_drafter {
  ngram_params p;
  std::vector<SeqState> seqs;
  std::string err;

  int fail(int code, const char* m) {
    err = m;
    return code;
  }
  bool valid(int32_t s) const { return s >= 0 && s < p.max_seqs; }

  void predict(const SeqState& st, std::vector<int32_t>& out) const {
    out.clear();
    int32_t a = st.prev2, b = st.prev1;
    while ((int)out.size() < p.max_drafts) {
      const Conts* c = nullptr;
      if (a >= 0 && b >= 0) {
        auto it = st.tri.find(pair_key(a, b));
        if (it != st.tri.end()) c = &it->second;
      }
      if (!c && b >= 0) {
        auto it = st.bi.find(b);
        if (it != st.bi.end()) c = &it->second;
      }
      if (!c) break;
      const int32_t t = c->best();
      out.push_back(t);
      a = b;
      b = t;
    }
  }

  int observe(int32_t s, const int32_t* tok, int32_t n) {
    if (!valid(s)) return fail(kEnoseq, "sequence id out of range");
    if (n < 0 || (n > 0 && !tok)) return fail(kEinval, "bad token array");
    for (int i = 0; i < n; ++i)
      if (tok[i] < 0) return fail(kEinval, "tokens must be >= 0");
    SeqState& st = seqs[s];
    if (n == 0) return 0;
    if (!st.pending.empty()) {
      size_t m = 0;
      while (m < st.pending.size() && m < (size_t)n && st.pending[m] == tok[m]) ++m;
      st.rate = (1.0 - p.ema_tau) * st.rate + p.ema_tau * ((double)m / (double)st.pending.size());
    }
    st.pending.clear();
    for (int i = 0; i < n; ++i) {
      const int32_t t = tok[i];
      if (st.prev1 >= 0) st.bi[st.prev1].add(t, st.seen);
      if (st.prev2 >= 0) st.tri[pair_key(st.prev2, st.prev1)].add(t, st.seen);
      st.prev2 = st.prev1;
      st.prev1 = t;
      ++st.seen;
    }
    return 0;
  }

  int draft(int32_t s, int32_t* out, int32_t* n_out) {
    SeqState& st = seqs[s];
    predict(st, st.pending);
    const bool on = st.rate >= p.ema_threshold;
    int32_t k = on ? (int32_t)st.pending.size() : 0;
    for (int i = 0; i < k; ++i) out[i] = st.pending[i];
    *n_out = k;
    return 0;
  }
};

extern "C" {

int ngram_create(const ngram_params* p, ngram_drafter** out) {
  if (!p || !out) return kEinval;
  *out = nullptr;
  if (p->max_seqs < 1 || p->max_drafts < 1 || p->max_drafts > kMaxDrafts) return kEinval;
  if (!(p->ema_tau > 0.0 && p->ema_tau <= 1.0) || !(p->ema_threshold >= 0.0 && p->ema_threshold <= 1.0))
    return kEinval;
  ngram_drafter* d = new ngram_drafter();
  d->p = *p;
  d->seqs.resize(p->max_seqs);
  *out = d;
  return 0;
}

int ngram_destroy(ngram_drafter* d) {
  delete d;
  return 0;
}

int ngram_observe(ngram_drafter* d, int32_t seq, const int32_t* tokens, int32_t n) {
  if (!d) return kEinval;
  return d->observe(seq, tokens, n);
}

int ngram_draft(ngram_drafter* d, int32_t seq, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!d) return kEinval;
  if (!d->valid(seq)) return d->fail(kEnoseq, "sequence id out of range");
  if (!out || !n_out || cap < d->p.max_drafts) return d->fail(kEinval, "out needs max_drafts entries");
  return d->draft(seq, out, n_out);
}

int ngram_draft_batch(ngram_drafter* d, int32_t n_seqs, const int32_t* seq_ids, int32_t* out, int32_t* n_out) {
  if (!d) return kEinval;
  if (n_seqs < 0 || (n_seqs > 0 && (!seq_ids || !out || !n_out))) return d->fail(kEinval, "bad arrays");
  for (int i = 0; i < n_seqs; ++i)
    if (!d->valid(seq_ids[i])) return d->fail(kEnoseq, "sequence id out of range");
  for (int i = 0; i < n_seqs; ++i) d->draft(seq_ids[i], out + (size_t)i * d->p.max_drafts, n_out + i);
  return 0;
}

int ngram_observe_batch(ngram_drafter* d, int32_t n_seqs, const int32_t* seq_ids, const int32_t* counts,
                        const int32_t* tokens) {
  if (!d) return kEinval;
  if (n_seqs < 0 || (n_seqs > 0 && (!seq_ids || !counts))) return d->fail(kEinval, "bad arrays");
  int64_t total = 0;
  for (int i = 0; i < n_seqs; ++i) {  // validate everything before changing anything
    if (!d->valid(seq_ids[i])) return d->fail(kEnoseq, "sequence id out of range");
    if (counts[i] < 0) return d->fail(kEinval, "counts must be >= 0");
    for (int j = 0; j < counts[i]; ++j)
      if (!tokens || tokens[total + j] < 0) return d->fail(kEinval, "tokens must be >= 0");
    total += counts[i];
  }
  int64_t off = 0;
  for (int i = 0; i < n_seqs; ++i) {
    d->observe(seq_ids[i], tokens + off, counts[i]);
    off += counts[i];
  }
  return 0;
}

int ngram_state(const ngram_drafter* d, int32_t seq, double* ema, int32_t* enabled, int64_t* observed) {
  if (!d) return kEinval;
  if (!d->valid(seq)) return kEnoseq;
  const SeqState& st = d->seqs[seq];
  if (ema) *ema = st.rate;
  if (enabled) *enabled = st.rate >= d->p.ema_threshold ? 1 : 0;
  if (observed) *observed = st.seen;
  return 0;
}

int ngram_reset(ngram_drafter* d, int32_t seq) {
  if (!d) return kEinval;
  if (!d->valid(seq)) return d->fail(kEnoseq, "sequence id out of range");
  d->seqs[seq] = SeqState();
  return 0;
}

const char* ngram_last_error(const ngram_drafter* d) { return d ? d->err.c_str() : "null handle"; }

}  // extern "C"
