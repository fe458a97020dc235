// kvcore.cpp - see kvcore.h.
#include "kvcore.h"

#include <cmath>
#include <cstring>

namespace svattn {

// ---- half precision --------------------------------------------------------

uint16_t half_bits_rne(double x, bool* sat) {
  uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  double a = std::fabs(x);
  if (std::isnan(a)) return 0x7E00;
  if (a >= 65520.0) {  // would round to infinity
    if (sat) *sat = true;
    return sign | 0x7BFF;
  }
  if (a < 0x1p-14) {  // subnormal (or zero): multiples of 2^-24
    double m = std::nearbyint(a * 0x1p24);
    return sign | (uint16_t)m;  // 1024 becomes the smallest normal, as it should
  }
  int e2;
  std::frexp(a, &e2);      // a = f * 2^e2, f in [0.5, 1)
  int e = e2 - 1;          // a in [2^e, 2^(e+1))
  double m = std::nearbyint(std::ldexp(a, 10 - e));  // in [1024, 2048]
  if (m == 2048.0) {
    m = 1024.0;
    e += 1;
  }
  if (e + 15 >= 31) {
    if (sat) *sat = true;
    return sign | 0x7BFF;
  }
  return sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)m - 1024);
}

double half_bits_to_double(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0)
    v = std::ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = std::ldexp((double)(f + 1024), e - 25);
  return s ? -v : v;
}

// ---- codec -----------------------------------------------------------------

static double normal_pdf(double x) {
  if (std::isinf(x)) return 0.0;
  return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
}
static double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

// Lloyd's two conditions, iterated: thresholds at the midpoints of adjacent
// levels; each level at the mean of N(0,1) restricted to its cell,
// (pdf(a) - pdf(b)) / (cdf(b) - cdf(a)).  Kept odd-symmetric each step.
void lloyd_max_gaussian8(double c[8], double t[7]) {
  for (int i = 0; i < 8; ++i) c[i] = -2.0 + 4.0 * i / 7.0;
  for (int it = 0; it < 200000; ++it) {
    double edge[9];
    edge[0] = -INFINITY;
    edge[8] = INFINITY;
    for (int i = 0; i < 7; ++i) edge[i + 1] = 0.5 * (c[i] + c[i + 1]);
    double nc[8];
    for (int i = 0; i < 8; ++i)
      nc[i] = (normal_pdf(edge[i]) - normal_pdf(edge[i + 1])) /
              (normal_cdf(edge[i + 1]) - normal_cdf(edge[i]));
    double step = 0.0;
    for (int i = 0; i < 8; ++i) {
      double v = 0.5 * (nc[i] - nc[7 - i]);
      step = std::fmax(step, std::fabs(v - c[i]));
      c[i] = v;
    }
    if (step < 1e-15) break;
  }
  for (int i = 0; i < 7; ++i) t[i] = 0.5 * (c[i] + c[i + 1]);
}

void make_codec(int d, uint64_t seed, Codec* out) {
  out->d = d;
  out->signs.assign(d, 1);
  out->s.assign((size_t)d * d, 0.f);
  SplitMix64 g(seed);
  for (int i = 0; i < d; ++i) out->signs[i] = (g.next() >> 63) ? -1 : 1;
  for (size_t t = 0; t < (size_t)d * d; t += 2) {
    uint64_t x1 = g.next(), x2 = g.next();
    double u1 = (double)((x1 >> 11) + 1) * 0x1p-53;
    double u2 = (double)(x2 >> 11) * 0x1p-53;
    double rho = std::sqrt(-2.0 * std::log(u1));
    out->s[t] = (float)(rho * std::cos(2.0 * M_PI * u2));
    out->s[t + 1] = (float)(rho * std::sin(2.0 * M_PI * u2));
  }
  lloyd_max_gaussian8(out->levels, out->thresholds);
  for (int i = 0; i < 8; ++i) {
    out->levels16_bits[i] = half_bits_rne(out->levels[i], nullptr);
    out->levels16[i] = half_bits_to_double(out->levels16_bits[i]);
  }
}

// ---- core ------------------------------------------------------------------

int Core::init(const CoreParams& p, std::string* err) {
  auto bad = [&](const char* m) {
    if (err) *err = m;
    return (int)EINVAL_;
  };
  if (p.num_kv_heads < 1) return bad("num_kv_heads must be >= 1");
  if (p.head_dim != 64 && p.head_dim != 128 && p.head_dim != 256) return bad("head_dim must be 64, 128 or 256");
  if (p.block_size != kBlock) return bad("block_size must be 256");
  if (p.num_blocks < 1) return bad("num_blocks must be >= 1");
  if (p.max_seqs < 1) return bad("max_seqs must be >= 1");
  if (p.max_blocks_per_seq < 1) return bad("max_blocks_per_seq must be >= 1");
  if ((int64_t)p.max_blocks_per_seq * kBlock > (int64_t)INT32_MAX) return bad("max_blocks_per_seq too large");
  if (p.format != FMT_FP32 && p.format != FMT_BF16 && p.format != FMT_TQ3) return bad("unknown format");
  if (p.ring_window < 0) return bad("ring_window must be >= 0");
  p_ = p;
  // Free list order: identity for seed 0, else Fisher-Yates with SplitMix64.
  std::vector<int32_t> order(p.num_blocks);
  for (int i = 0; i < p.num_blocks; ++i) order[i] = i;
  if (p.alloc_seed != 0) {
    SplitMix64 g(p.alloc_seed);
    for (int i = p.num_blocks - 1; i >= 1; --i) {
      uint64_t j = g.next() % (uint64_t)(i + 1);
      std::swap(order[i], order[j]);
    }
  }
  free_.assign(order.rbegin(), order.rend());  // back() = order[0]
  table_.assign((size_t)p.max_seqs * p.max_blocks_per_seq, -1);
  owned_.assign(p.max_seqs, 0);
  first_.assign(p.max_seqs, 0);
  len_.assign(p.max_seqs, 0);
  if (p.format == FMT_TQ3) make_codec(p.head_dim, p.codec_seed, &codec_);
  return OK;
}

int Core::plan_append(int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new, AppendPlan* plan,
                      std::string* err, const int32_t* slack) const {
  auto fail = [&](int code, const std::string& m) {
    if (err) *err = m;
    return code;
  };
  if (n_seqs < 0) return fail(EINVAL_, "n_seqs < 0");
  if (n_seqs > 0 && (!seq_ids || !n_new)) return fail(EINVAL_, "null seq_ids / n_new");
  plan->segs.clear();
  plan->popped.clear();
  plan->table_index.clear();
  plan->released.clear();
  plan->released_index.clear();
  plan->total_rows = 0;
  std::vector<char> seen(p_.max_seqs, 0);
  for (int i = 0; i < n_seqs; ++i) {  // entries checked in call order
    int32_t s = seq_ids[i];
    if (!valid_seq(s)) return fail(ENOSEQ_, "sequence id " + std::to_string(s) + " out of range");
    if (seen[s]) return fail(EINVAL_, "sequence id " + std::to_string(s) + " repeated");
    seen[s] = 1;
    if (n_new[i] < 0) return fail(EINVAL_, "n_new < 0");
    int64_t len = (int64_t)len_[s] + n_new[i];
    int64_t blocks = (len + kBlock - 1) / kBlock;
    if (blocks > p_.max_blocks_per_seq)
      return fail(ERANGE_, "sequence " + std::to_string(s) + " would exceed max_blocks_per_seq");
  }
  // Walk the entries on a virtual free list: a ring cache's released blocks
  // go to its front (the vector's back) before the entry's pops.
  std::vector<int32_t> pushed;
  size_t k = free_.size();
  for (int i = 0; i < n_seqs; ++i) {
    const int32_t s = seq_ids[i];
    const int64_t len = (int64_t)len_[s] + n_new[i];
    const int32_t blocks = (int32_t)((len + kBlock - 1) / kBlock);
    int32_t keep = first_[s];
    if (p_.ring_window > 0) {
      const int64_t low = len - (slack ? slack[i] : 0);
      keep = std::max<int32_t>(keep, (int32_t)(std::max<int64_t>(0, low - kRingHistory - p_.ring_window + 1) / kBlock));
    }
    AppendSeg g{s, len_[s], n_new[i], (int32_t)plan->total_rows, 0, 0, keep};
    for (int32_t b = first_[s]; b < std::min(keep, owned_[s]); ++b) {
      const int32_t blk = table_[(size_t)s * p_.max_blocks_per_seq + b];
      pushed.push_back(blk);
      plan->released.push_back(blk);
      plan->released_index.push_back(s * p_.max_blocks_per_seq + b);
      ++g.released;
    }
    for (int32_t b = std::max(owned_[s], keep); b < blocks; ++b) {
      int32_t blk;
      if (!pushed.empty()) {
        blk = pushed.back();
        pushed.pop_back();
      } else if (k > 0) {
        blk = free_[--k];
      } else {
        return fail(ENOMEM_, "pool exhausted: not enough free blocks for the call (" +
                                 std::to_string(free_.size()) + " free)");
      }
      plan->popped.push_back(blk);
      plan->table_index.push_back(s * p_.max_blocks_per_seq + b);
      ++g.new_blocks;
    }
    plan->segs.push_back(g);
    plan->total_rows += n_new[i];
  }
  return OK;
}

void Core::commit_append(const AppendPlan& plan) {
  size_t i = 0, r = 0;
  for (const AppendSeg& g : plan.segs) {
    for (int b = 0; b < g.released; ++b, ++r) {
      free_.push_back(plan.released[r]);
      table_[plan.released_index[r]] = -1;
    }
    for (int b = 0; b < g.new_blocks; ++b, ++i) {
      free_.pop_back();
      table_[plan.table_index[i]] = plan.popped[i];
    }
    const int64_t len = (int64_t)g.pos0 + g.n;
    owned_[g.seq] = std::max<int32_t>(owned_[g.seq], (int32_t)((len + kBlock - 1) / kBlock));
    first_[g.seq] = g.keep_first;
    len_[g.seq] = (int32_t)len;
  }
}

int Core::rollback(int32_t seq, int32_t r, std::string* err) {
  if (!valid_seq(seq)) {
    if (err) *err = "sequence id out of range";
    return ENOSEQ_;
  }
  if (r < 0) {
    if (err) *err = "rollback count < 0";
    return EINVAL_;
  }
  if (r > len_[seq]) {
    if (err) *err = "rollback beyond seq_len";
    return ERANGE_;
  }
  if (!window_intact(seq, (int64_t)len_[seq] - r)) {
    if (err) *err = "rollback would reach positions a ring cache released";
    return ERANGE_;
  }
  len_[seq] -= r;
  return OK;
}

int Core::free_seq(int32_t seq, std::string* err) {
  if (!valid_seq(seq)) {
    if (err) *err = "sequence id out of range";
    return ENOSEQ_;
  }
  int32_t* row = &table_[(size_t)seq * p_.max_blocks_per_seq];
  for (int b = owned_[seq] - 1; b >= first_[seq]; --b) {
    free_.push_back(row[b]);  // last pushed = the first held block = next handed out
    row[b] = -1;
  }
  owned_[seq] = 0;
  first_[seq] = 0;
  len_[seq] = 0;
  return OK;
}

int Core::seq_len(int32_t seq, int32_t* out) const {
  if (!valid_seq(seq)) return ENOSEQ_;
  *out = len_[seq];
  return OK;
}

int Core::owned(int32_t seq, int32_t* out) const {
  if (!valid_seq(seq)) return ENOSEQ_;
  *out = owned_[seq];
  return OK;
}

}  // namespace svattn
