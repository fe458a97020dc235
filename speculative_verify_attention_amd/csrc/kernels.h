// kernels.h - launch arguments and host launchers of the gfx950 kernels.
// Arguments travel by value in the kernel-argument segment, so the host's
// values are captured when a launch is enqueued: no staging buffers, no
// host-to-device copies on the step path.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace svattn {

// ---- pool layout -------------------------------------------------------------
//
// One block holds 256 token positions of every kv head.
//  FP32/BF16 (e = element bytes):
//    K: [hkv][256][d]                        at 0
//    V: [hkv][4][d][64]                      at hkv*256*d*e
//  TQ3:
//    K codes  [hkv][256][d/2]  (nibble = code | sign << 3, dim i in nibble i)
//    K n16    [hkv][256]  fp16
//    K g16    [hkv][256]  fp16
//    V codes  [hkv][4][d][24 bytes]  (64 tokens x 3 bits, token t at bits 3t)
//    V n16    [hkv][256]  fp16
struct PoolLayout {
  int32_t fmt, hkv, d;
  int64_t block_bytes;
  int64_t k_off, v_off;            // FP32/BF16
  int64_t kc_off, kn_off, kg_off;  // TQ3
  int64_t vc_off, vn_off;          // TQ3
};

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
constexpr int kMaxAttnSeqs = 128;
constexpr int kTileKeys = 64;  // keys per wave iteration

struct AttnArgs {
  const uint8_t* pool;
  const int32_t* table;
  const float* q;    // [rows][hq][d] (TQ3: q' and q'' in the workspace instead)
  const float* q2;   // TQ3: q'' (S Pi q)
  float* out;        // [rows][hq][d]
  float* part;       // partial slots
  PoolLayout lay;
  int32_t hq, g, max_bps, window;
  float scale;       // multiplies <q, k>
  float softcap;     // 0 = off
  float inv_softcap;
  float qjl_coef;    // TQ3: sqrt(pi/2) / d
  float inv_sqrt_d;  // TQ3
  int32_t n_seqs;
  int32_t tiles_per_wg;
  int32_t total_tiles;
  int32_t n_wg;
  int32_t slot_stride;    // floats per partial slot
  int32_t rpad;           // padded rows per slot (32 * NCT)
  int32_t force_partial;  // 1: every pair goes through the merge
  int32_t pad0;
  uint16_t lev16_bits[8];
  int32_t seq[kMaxAttnSeqs];
  int32_t len[kMaxAttnSeqs];
  int32_t qrow0[kMaxAttnSeqs];
  int32_t nrows[kMaxAttnSeqs];
  int32_t tile_base[kMaxAttnSeqs + 1];  // prefix over sequences of hkv * tiles
};

struct QPrepArgs {
  const float* q;   // [rows][hq][d]
  float* q1;        // Pi q
  float* q2;        // S Pi q
  const int8_t* signs;
  const float* s_t;
  int32_t n_vec, d;
};

static_assert(sizeof(AttnArgs) <= 4096, "kernel arguments must fit the 4 KiB argument segment");
static_assert(sizeof(AppendArgs) <= 4096, "kernel arguments must fit the 4 KiB argument segment");
static_assert(sizeof(TableUpdateArgs) <= 4096, "kernel arguments must fit the 4 KiB argument segment");

hipError_t launch_attn(const AttnArgs& a, int nct, hipStream_t s);
hipError_t launch_merge(const AttnArgs& a, int nct, hipStream_t s);
hipError_t launch_qprep(const QPrepArgs& a, hipStream_t s);

}  // namespace svattn
