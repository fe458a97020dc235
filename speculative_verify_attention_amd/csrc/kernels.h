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

// Keys per attention tile (one wavefront iteration): 16 KiB of bf16 K and V
// at d <= 128, one 32-key sub-tile otherwise.
constexpr int tile_keys(int fmt, int d) { return fmt == 1 ? 32 * (128 / d > 1 ? 128 / d : 1) : fmt == 0 ? 32 : 64; }

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

// A call's work is cut into chunks of consecutive tiles of one (sequence, kv
// head) pair; workgroup w takes one chunk.  Sequence i's pairs are split into
// ksplit[i] chunks each, and its workgroups are wg_base[i] .. wg_base[i+1]-1
// (kv head major).  A pair split into more than one chunk leaves one partial
// slot per chunk (slot index = workgroup index) for the merge.
struct AttnArgs {
  const uint8_t* pool;
  const int32_t* table;
  const float* q;    // [rows][hq][d] (TQ3: q' = Pi q)
  const float* q2;   // TQ3: q'' = S Pi q
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
  int32_t n_wg;
  int32_t slot_stride;    // floats per partial slot
  int32_t rpad;           // padded rows per slot (32 * NCT)
  int32_t force_partial;  // 1: every pair goes through the merge
  int32_t tile_keys;      // keys per tile (tile_keys(fmt, d))
  uint16_t lev16_bits[8];
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

static_assert(sizeof(AttnArgs) <= 4096, "kernel arguments must fit the 4 KiB argument segment");
static_assert(sizeof(AppendArgs) <= 4096, "kernel arguments must fit the 4 KiB argument segment");
static_assert(sizeof(TableUpdateArgs) <= 4096, "kernel arguments must fit the 4 KiB argument segment");

hipError_t launch_attn(const AttnArgs& a, int nct, hipStream_t s);
hipError_t launch_merge(const AttnArgs& a, int nct, hipStream_t s);
hipError_t launch_qprep(const QPrepArgs& a, hipStream_t s);

}  // namespace svattn
