// kvcore.h - HIP-free host core of the KV cache: block allocator, per-sequence
// block tables, seq_len, all-or-nothing append reservation, O(1) rollback, and
// the compressed-cache codec constants.  Builds with plain g++ so the host
// logic can be tested without a GPU; libsvattn links it unchanged.
//
// Behaviour follows the AX Engine page, "Core Technical Architecture &
// Methods" (deterministic, synchronous block manager; slice-update appends
// into preallocated buffers; rollback moves the length pointer only) and the
// mlx-engine blog's prompt-caching section (256-token blocks).
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

namespace svattn {

constexpr int kBlock = 256;
constexpr int kMaxRows = 8;
// A ring cache keeps the last window + kRingHistory positions of a sequence:
// the rows one verify call appends can still be verified and rolled back.
constexpr int kRingHistory = kMaxRows;

enum Status { OK = 0, EINVAL_ = -1, ENOMEM_ = -2, ERANGE_ = -3, ENOSEQ_ = -4, EDEVICE_ = -5 };
enum Format { FMT_FP32 = 0, FMT_BF16 = 1, FMT_TQ3 = 2 };

struct CoreParams {
  int32_t num_kv_heads = 0;
  int32_t head_dim = 0;
  int32_t block_size = kBlock;
  int32_t num_blocks = 0;
  int32_t max_seqs = 0;
  int32_t max_blocks_per_seq = 0;
  int32_t format = FMT_BF16;
  int32_t ring_window = 0;  // > 0: ring cache for layers whose window is at most this
  uint64_t alloc_seed = 0;
  uint64_t codec_seed = 0;
};

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014; the 64-bit form of Vigna's
// splitmix64.c): golden-gamma increment, two xor-shift-multiply rounds, a
// final xor-shift.
struct SplitMix64 {
  uint64_t state;
  explicit SplitMix64(uint64_t seed) : state(seed) {}
  uint64_t next() {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

// Round to IEEE half, nearest-even, saturating at 65504 (sets *sat).
uint16_t half_bits_rne(double x, bool* sat);
double half_bits_to_double(uint16_t h);

// Codec constants of the compressed format (SwiftLM page, TurboQuant
// KV-cache compression passage: Lloyd-Max codes, rotation, 1-bit QJL).
struct Codec {
  int d = 0;
  std::vector<int8_t> signs;   // D, +-1
  std::vector<float> s;        // S, d x d row-major, N(0,1)
  double levels[8];            // Lloyd-Max centroids for N(0,1)
  double levels16[8];          // fp16-rounded levels (the stored reconstruction levels)
  uint16_t levels16_bits[8];
  double thresholds[7];        // decision thresholds (midpoints of the centroids)
};

// Lloyd-Max 8-level quantizer for N(0,1) by fixed-point iteration.
void lloyd_max_gaussian8(double levels[8], double thresholds[7]);
void make_codec(int d, uint64_t seed, Codec* out);

// One sequence's part of an append plan.
struct AppendSeg {
  int32_t seq;
  int32_t pos0;       // seq_len before the append
  int32_t n;          // new positions
  int32_t src_row0;   // first source row in the caller's K/V
  int32_t new_blocks; // blocks popped for this sequence
  int32_t released;   // blocks a ring cache releases first
  int32_t keep_first; // first kept block after the append (0 for plain caches)
};

struct AppendPlan {
  std::vector<AppendSeg> segs;
  std::vector<int32_t> popped;           // blocks popped, in order, all sequences
  std::vector<int32_t> table_index;      // flat table index for each popped block
  std::vector<int32_t> released;         // ring caches: blocks released, in order
  std::vector<int32_t> released_index;   // flat table index of each
  int64_t total_rows = 0;
};

class Core {
 public:
  int init(const CoreParams& p, std::string* err);
  const CoreParams& params() const { return p_; }

  // Validate an append and compute what it would do, without changing state.
  // slack (optional, per entry): how far below the host's length the true
  // length may be (rollbacks still pending on the device); a ring cache then
  // keeps that much more history.
  int plan_append(int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new, AppendPlan* plan,
                  std::string* err, const int32_t* slack = nullptr) const;
  // Apply a plan made against the current state.
  void commit_append(const AppendPlan& plan);

  int rollback(int32_t seq, int32_t r, std::string* err);
  int free_seq(int32_t seq, std::string* err);

  int seq_len(int32_t seq, int32_t* out) const;
  // Table entries in use (the index one past the last held block; ring
  // caches hold only entries from first_block on, the rest read -1).
  int owned(int32_t seq, int32_t* out) const;
  int32_t first_block(int32_t seq) const { return first_[seq]; }
  // Ring caches: can a window still see everything it needs once the
  // sequence is at `len` positions?  (Always true for plain caches.)
  bool window_intact(int32_t seq, int64_t len) const {
    return p_.ring_window == 0 || std::max<int64_t>(0, len - p_.ring_window + 1) >= (int64_t)first_[seq] * kBlock;
  }
  const int32_t* table_row(int32_t seq) const { return &table_[(size_t)seq * p_.max_blocks_per_seq]; }
  int32_t free_count() const { return (int32_t)free_.size(); }
  bool valid_seq(int32_t seq) const { return seq >= 0 && seq < p_.max_seqs; }
  const Codec& codec() const { return codec_; }

 private:
  CoreParams p_;
  std::vector<int32_t> free_;   // stack: free_.back() is the front of the free list
  std::vector<int32_t> table_;  // max_seqs x max_blocks_per_seq
  std::vector<int32_t> owned_;  // table entries in use per sequence
  std::vector<int32_t> first_;  // first held table entry (ring caches)
  std::vector<int32_t> len_;    // seq_len per sequence
  Codec codec_;
};

}  // namespace svattn
