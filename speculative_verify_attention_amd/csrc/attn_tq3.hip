// attn_tq3.hip - verify attention over the compressed (TQ3) cache on gfx950:
// the query rotation and the dequantize-inside-attention partial kernel.
//
// SwiftLM page, TurboQuant KV-cache compression passage: keys are 3-bit
// Lloyd-Max codes plus a 1-bit QJL residual, values 3-bit codes; the codes
// are dequantized inside the attention kernel.  The scores use the factored
// form of the decoded key,
//   <q, k> = n16/sqrt(d) <q', c16[code]> + g16 sqrt(pi/2)/d <q'', b>,
// with q' = Pi q and q'' = S q' computed once per query (the rotation is
// applied to the few queries, not to the many keys); values are accumulated
// in the rotated frame with their norm folded into the probability, and the
// merge rotates the result back (o = Pi^T o').
//
// Precision.  The code levels c16 and the signs are exact in fp16; q', q''
// and the probabilities are carried as two fp16 parts each (hi + lo, about
// 2^-22 relative), so every product runs as two v_mfma_f32_32x32x16_f16 with
// fp32 accumulation (48 matrix-core instructions per 32-key sub-tile).  One
// part is not enough: its 2^-11 rounding of the query moves a peaked softmax
// by about 1e-3.
//
// Layout and work split follow the plain kernel: one chunk of 32-key
// sub-tiles of one (sequence, kv head) per workgroup, eight waves (two per
// SIMD, so that one wave's table reads and matrix-core latency hide behind
// the other's work), keys as the MFMA M dimension.  Every wave-wide load
// reads contiguous memory: 1 KiB per 4 key k-steps, 768 B per two value
// d-tiles, and the 192-byte scales.  Codes become fp16 operands through two
// small LDS tables: one byte of key nibbles -> (2 levels, 2 signs), 6 bits of
// value codes -> 2 levels.
#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "kernels.h"
#include "qprep.h"

// Query-fragment parts held in registers (the others are read from LDS at
// every use: the register budget of two waves per SIMD) and the depth of the
// sub-tile ring.
#ifndef SVATTN_TQ3_QREGS
#define SVATTN_TQ3_QREGS 1
#endif
#ifndef SVATTN_TQ3_NBUF
#define SVATTN_TQ3_NBUF 2
#endif
// Waves per workgroup (one workgroup per CU: the tables fill the LDS).
#ifndef SVATTN_TQ3_WAVES
#define SVATTN_TQ3_WAVES 8
#endif
// Non-temporal hint on the sub-tile loads.
#ifndef SVATTN_TQ3_NT
#define SVATTN_TQ3_NT 1
#endif

namespace svattn {

// Waves per workgroup and query-fragment parts (q' hi, q'' hi, q' lo,
// q'' lo) held in registers, d <= 128: two waves per SIMD, the first part in
// registers as well as all four in LDS (the others are read from LDS at
// every use).  (d = 256 runs on wave pairs: attn_tq3_pair_kernel.)
template <int D>
struct TQ3Cfg {
  static_assert(D <= 128, "d = 256 runs on wave pairs");
  static constexpr int NW = SVATTN_TQ3_WAVES;
  static constexpr int NREG = SVATTN_TQ3_QREGS;
  static constexpr int LDS_PART0 = 0;  // the first part kept in LDS
  static constexpr int NPART_LDS = 4 - LDS_PART0;
};

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Two-part fp16 split of a pair of floats, x = hi + lo to ~2^-21: hi is one
// explicit conversion (toward zero), and the residual is taken from that
// same value.  Written as (_Float16)x and x - (float)(_Float16)x the compiler
// may emit two conversions for hi (a scalar one for the residual and a
// packed one for the operand) that round exact fp16 ties differently, and
// the two parts then miss x by one fp16 ulp.
__device__ __forceinline__ u32x2_t split_f16_pair(float a, float b) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(a, b);
  const float ra = a - (float)h[0], rb = b - (float)h[1];
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t l = {(_Float16)ra, (_Float16)rb};
  return u32x2_t{__builtin_bit_cast(uint32_t, h), __builtin_bit_cast(uint32_t, l)};  // (hi pair, lo pair)
}

// The same split of two products p * n (n an fp16 value widened): hi from the
// rounded product, lo the exact product less hi rounded once (one fma), so
// that hi + lo carries the product to ~2^-21.  Each product and residual is
// one mixed-precision fma that reads n as fp16.
__device__ __forceinline__ u32x2_t split_f16_prod(float p0, float n0, float p1, float n1) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(fmaf(p0, n0, 0.0f), fmaf(p1, n1, 0.0f));
  const float ra = fmaf(p0, n0, -(float)h[0]), rb = fmaf(p1, n1, -(float)h[1]);
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t l = {(_Float16)ra, (_Float16)rb};
  return u32x2_t{__builtin_bit_cast(uint32_t, h), __builtin_bit_cast(uint32_t, l)};
}

// ---- query rotation ---------------------------------------------------------------

// One wave per query vector (qprep_vector in qprep.h), four per workgroup.
template <int D>
__global__ __launch_bounds__(256) void qprep_kernel(QPrepArgs a) {
  __shared__ float buf[4][D];
  const int wave = threadIdx.x >> 6;
  const int64_t vec = (int64_t)blockIdx.x * 4 + wave;
  if (vec >= a.n_vec) return;
  qprep_vector<D>(a, vec, buf[wave]);
}

hipError_t launch_qprep(const QPrepArgs& a, hipStream_t s) {
  if (a.n_vec <= 0) return hipSuccess;
  dim3 grid((a.n_vec + 3) / 4);
  if (a.d == 64)
    hipLaunchKernelGGL(qprep_kernel<64>, grid, dim3(256), 0, s, a);
  else if (a.d == 128)
    hipLaunchKernelGGL(qprep_kernel<128>, grid, dim3(256), 0, s, a);
  else if (a.d == 256)
    hipLaunchKernelGGL(qprep_kernel<256>, grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---- the partial kernel ----------------------------------------------------------

// Raw bytes of one 32-key sub-tile for this lane.
template <int D>
struct TQ3Regs {
  u32x4_t kc[D / 64];     // key nibbles, 4 k-steps per plane
  uint32_t vc[D / 64][3]; // value codes, 2 d-tiles per plane
  uint32_t sc;            // scales dword `lane` (lanes 0..47)
};

template <int D>
__device__ __forceinline__ void load_tq3(TQ3Regs<D>& t, const uint8_t* __restrict__ sub, int lane) {
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    const uint8_t* vp = sub + 16 * D + j * 768 + lane * 12;
    if constexpr (SVATTN_TQ3_NT) {
      t.kc[j] = ld_stream(sub + j * 1024 + lane * 16);
      t.vc[j][0] = ld_stream_u32(vp);
      t.vc[j][1] = ld_stream_u32(vp + 4);
      t.vc[j][2] = ld_stream_u32(vp + 8);
    } else {
      t.kc[j] = *reinterpret_cast<const u32x4_t*>(sub + j * 1024 + lane * 16);
      t.vc[j][0] = reinterpret_cast<const uint32_t*>(vp)[0];
      t.vc[j][1] = reinterpret_cast<const uint32_t*>(vp)[1];
      t.vc[j][2] = reinterpret_cast<const uint32_t*>(vp)[2];
    }
  }
  // lanes 48..63 repeat lanes 32..47 (no branch around the load)
  const uint8_t* sp = sub + 28 * D + (lane < 48 ? lane : lane - 16) * 4;
  if constexpr (SVATTN_TQ3_NT)
    t.sc = ld_stream_u32(sp);
  else
    t.sc = *reinterpret_cast<const uint32_t*>(sp);
}

// Shared memory of the partial kernel (NW waves; 8 = two per SIMD).
//  * key table, indexed by (byte of two key nibbles, lane slot): every lane of
//    a 32-lane group reads its own dword column (levels in the row's first
//    half, signs in the second), so table reads never conflict on LDS banks
//    whatever the codes are;
//  * query fragments: per column group, the fp16 parts of q' and q'' in the
//    matrix-core operand order, [part][k-step][lane] x 16 bytes, shared by
//    the column group's waves;
//  * value table (6 bits of codes -> 2 levels), also one copy per lane slot
//    (a single copy puts entries e and e + 32 on one bank), and per-wave
//    scale slices.
// The combine buffer reuses the key table and fragments after the loop.
template <int D, int NCT>
struct TQ3Smem {
  static constexpr int NW = TQ3Cfg<D>::NW;
  static constexpr int TL = NW / NCT;
  static constexpr int NPART = TQ3Cfg<D>::NPART_LDS;  // parts in LDS (of q' hi, q'' hi, q' lo, q'' lo)
  // below 64 KiB: value table, scale slices, query fragments; the key table
  // fills the next 64 KiB, so that a key-table address is one byte permute
  // of (slot, code byte, 1) and every other address fits an instruction's
  // 16-bit offset field
  static constexpr int VLUT_OFF = 0;     // 64 entries x 32 lane slots x 4 bytes
  static constexpr int SCL_OFF = 8192;  // per wave: two slots of 48 dwords, alternating between sub-tiles
  static constexpr int QF_OFF = (SCL_OFF + NW * 2 * 48 * 4 + 4095) / 4096 * 4096;
  static constexpr int QF_CT_BYTES = NPART * (D / 16) * 64 * 16;
  static constexpr int KLUT_OFF = 65536;  // row = code byte: 32 level slots, then 32 sign slots
  // a second column group's fragments go above the key table when both do
  // not fit below it (two-part fragments of 64 KiB for d = 128)
  static constexpr bool LOW2 = QF_OFF + NCT * QF_CT_BYTES <= KLUT_OFF;
  static constexpr int qf_off(int ct) { return (LOW2 || ct == 0) ? QF_OFF + ct * QF_CT_BYTES : KLUT_OFF + 65536; }
  static constexpr int BYTES = (LOW2 || NCT == 1) ? KLUT_OFF + 65536 : KLUT_OFF + 65536 + QF_CT_BYTES;
  static_assert(SCL_OFF + NW * 2 * 48 * 4 <= QF_OFF, "scale slices");
  static_assert(QF_OFF + QF_CT_BYTES <= KLUT_OFF, "query fragments");
  static_assert(BYTES <= 160 * 1024, "LDS of one workgroup");
  static constexpr int CBUF_OFF = QF_OFF;  // the combine buffer reuses fragments and key table
  static_assert(CBUF_OFF + CombineBuf<D, NCT, NW>::FLOATS * 4 <= BYTES, "combine buffer");
};

// LDS address of part `part`, k-step kk, of a lane's query fragments (P0:
// the first part kept in LDS).
template <int D, int P0 = TQ3Cfg<D>::LDS_PART0>
__device__ __forceinline__ int qfrag_off(int part, int kk, int lane) {
  return ((part - P0) * (D / 16) + kk) * 1024 + lane * 16;
}
template <int D, int P0 = TQ3Cfg<D>::LDS_PART0>
__device__ __forceinline__ f16x8_t qfrag(const uint8_t* qf, int part, int kk, int lane) {
  return *reinterpret_cast<const f16x8_t*>(qf + qfrag_off<D, P0>(part, kk, lane));
}

// Query fragments of one lane: the leading NREG parts in registers, the
// others read from LDS at every use.  P0: the first part kept in LDS (0:
// every part is there, the register parts being copies; NREG: the register
// parts are not in LDS and the prologue fills them itself).
template <int D, int NREG_ = TQ3Cfg<D>::NREG, int P0 = TQ3Cfg<D>::LDS_PART0>
struct QFrags {
  static constexpr int NREG = NREG_;
  static constexpr int NR = NREG > 0 ? NREG : 1;
  f16x8_t f[NR][D / 16];
  const uint8_t* qf;
  int lane;
  __device__ __forceinline__ void init(const uint8_t* q, int l) {
    qf = q;
    lane = l;
    if constexpr (P0 == 0) {
#pragma unroll
      for (int pt = 0; pt < NREG; ++pt)
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) f[pt][kk] = qfrag<D, P0>(qf, pt, kk, lane);
    }
  }
  __device__ __forceinline__ f16x8_t get(int pt, int kk) const {
    if (pt < NREG)
      return f[pt < NR ? pt : 0][kk];
    else
      return qfrag<D, P0>(qf, pt, kk, lane);
  }
};

struct NoScoreHook {
  __device__ __forceinline__ void operator()(float (&)[16]) const {}
};

// scores(p) gets the sub-tile's scores before any non-linear step (the
// multiplier's fold, the soft cap, the mask): the two-wave d = 256 kernel
// adds the other half's partial scores there.
template <int D, bool CAP, typename QF, typename ScoreHook = NoScoreHook>
__device__ __forceinline__ void process_tq3(ColState<D>& cs, const TQ3Regs<D>& t, const QF& qr,
                                            const uint8_t* __restrict__ lds, const uint32_t* __restrict__ vlut,
                                            uint32_t* scl, const AttnArgs& a, int key0, int L, int n, int ppos,
                                            int lane, uint32_t kslot, ScoreHook scores = ScoreHook()) {
  const int hh = lane >> 5;
  // scl: this sub-tile's scales (K norm, K residual norm, V norm), written
  // to the wave's LDS slot during the previous sub-tile
  auto scale_words = [&](int f, uint32_t(&wd)[8]) {
    const u32x4_t x0 = reinterpret_cast<const u32x4_t*>(scl)[(hh * 3 + f) * 2];
    const u32x4_t x1 = reinterpret_cast<const u32x4_t*>(scl)[(hh * 3 + f) * 2 + 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wd[j] = x0[j];
      wd[4 + j] = x1[j];
    }
  };
  auto half_at = [](const uint32_t(&wd)[8], int r) -> float {
    const uint32_t w = wd[r >> 1];
    return (float)__builtin_bit_cast(_Float16, (uint16_t)((r & 1) ? (w >> 16) : (w & 0xFFFF)));
  };

  // S1 = <q', c16[code]>, S2 = <q'', b> for the 32 keys of the sub-tile.
  // Byte b of a nibble word selects the table row, the lane's slot the
  // column: address = 65536 + byte * 256 + slot * 4 (+ 128 for the signs),
  // assembled from the bytes of (kslot, w) by one permute per read, so the
  // reads land directly in the operand registers.  The reads of k-step
  // kk + 1 are issued before the products of k-step kk.
  auto fetch = [&](int kk, u32x4_t& mse, u32x4_t& qjl) {
    const uint32_t w = t.kc[kk >> 2][kk & 3];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t sel = 0x0C020000u | ((4u + b) << 8);
      mse[b] = *reinterpret_cast<const uint32_t*>(lds + __builtin_amdgcn_perm(w, kslot, sel));
      qjl[b] = *reinterpret_cast<const uint32_t*>(lds + __builtin_amdgcn_perm(w, kslot | 0x80u, sel));
    }
  };
  f32x16_t s1 = {}, s2 = {};
  u32x4_t mse[2], qjl[2];
  // issue priority by phase: highest for the key products, lowest for the
  // softmax, so that the other wave of the SIMD fills the matrix-core phases
  // with its vector work
  __builtin_amdgcn_s_setprio(2);
  fetch(0, mse[0], qjl[0]);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (kk + 1 < D / 16) fetch(kk + 1, mse[(kk + 1) & 1], qjl[(kk + 1) & 1]);
    const f16x8_t km = __builtin_bit_cast(f16x8_t, mse[kk & 1]), kq = __builtin_bit_cast(f16x8_t, qjl[kk & 1]);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(km, qr.get(0, kk), s1, 0, 0, 0);
    s2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(kq, qr.get(1, kk), s2, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(km, qr.get(2, kk), s1, 0, 0, 0);
    s2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(kq, qr.get(3, kk), s2, 0, 0, 0);
  }
  __builtin_amdgcn_s_setprio(0);
  // scores in log2 units (q'' already carries the QJL coefficient relative
  // to the first term), times 1 / smul: without a soft cap and with a
  // positive multiplier, the multiplier is left to the softmax, which folds
  // it into the exponent's argument
  const bool fold = !CAP && a.q1_mul > 0.0f;
  const float smul = fold ? a.q1_mul : 1.0f;
  float p[1][16];
  {
    uint32_t nw[8], gw[8];
    scale_words(0, nw);
    scale_words(1, gw);
#pragma unroll
    for (int r = 0; r < 16; ++r) p[0][r] = fmaf(s2[r], half_at(gw, r), fmaf(s1[r], half_at(nw, r), 0.0f));
    scores(p[0]);
    if (!fold) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = p[0][r] * a.q1_mul;
        if constexpr (CAP) x = a.cap_l2 * tanh_nb(x * a.inv_cap_l2);
        p[0][r] = x;
      }
    }
  }
  uint32_t vw[8];
  scale_words(2, vw);
  __builtin_amdgcn_wave_barrier();
  const bool full = key0 + 32 <= L - n + 1 && (a.window == 0 || L - key0 <= a.window);
  if (!full) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kp = key0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      const bool vis = kp <= ppos && (a.window == 0 || ppos - kp < a.window);
      p[0][r] = vis ? p[0][r] : NEG_INF;
      // slots past the end of the sequence may hold any bits: zero their norm
      if (kp >= L) vw[r >> 1] &= (r & 1) ? 0x0000FFFFu : 0xFFFF0000u;
    }
  }
  // The probabilities carry the value norms into fp16 products: they may
  // reach the lazy reference's 2^8 only while every value norm of the
  // sub-tile is at most 240, else the reference moves to the sub-tile's
  // maximum (probabilities <= 1), so that p * n16v stays finite.  The norms
  // are non-negative fp16 (saturated at 65504), which order as 16-bit
  // integers: 240 is 0x5B80.  Every lane holds the norms of half the
  // sub-tile's keys, so one ballot over the wave covers all of them.
  typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
  u16x2_t nv[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) nv[q] = __builtin_bit_cast(u16x2_t, vw[q]);
#pragma unroll
  for (int w = 4; w >= 1; w >>= 1)  // tree: no chain of dependent packed operations
#pragma unroll
    for (int q = 0; q < w; ++q) nv[q] = __builtin_elementwise_max(nv[q], nv[q + w]);
  const u16x2_t nv2 = nv[0];
  const bool big = __builtin_amdgcn_ballot_w64(nv2[0] > 0x5B80u || nv2[1] > 0x5B80u) != 0;
  softmax_update<D, 1>(cs, p, big ? 0.0f : 8.0f, smul);
  __builtin_amdgcn_s_setprio(1);
  // O'^T += C16[vcode]^T (P * n16v)^T; the merge applies 1/sqrt(d)
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    u32x4_t phw, plw;  // fp16 pairs
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int r = 8 * v + e;
      const u32x2_t sp = split_f16_prod(p[0][r], half_at(vw, r), p[0][r + 1], half_at(vw, r + 1));
      phw[e / 2] = sp[0];
      plw[e / 2] = sp[1];
    }
    const f16x8_t phi = __builtin_bit_cast(f16x8_t, phw), plo = __builtin_bit_cast(f16x8_t, plw);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const uint32_t* w3 = t.vc[dt >> 1];
      // 24 bits of codes: d-tile dt, keys of k-step v
      uint32_t g;
      if ((dt & 1) == 0)
        g = v == 0 ? w3[0] : __builtin_amdgcn_alignbit(w3[1], w3[0], 24);
      else
        g = v == 0 ? __builtin_amdgcn_alignbit(w3[2], w3[1], 16) : (w3[2] >> 8);
      u32x4_t vv;
#pragma unroll
      for (int q = 0; q < 4; ++q) vv[q] = vlut[((g >> (6 * q)) & 63) << 5];
      const f16x8_t vop = __builtin_bit_cast(f16x8_t, vv);
      cs.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, phi, cs.acc[dt], 0, 0, 0);
      cs.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, plo, cs.acc[dt], 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

template <int D, int NCT, bool CAP>
__global__ __launch_bounds__(TQ3Cfg<D>::NW * 64) void attn_tq3_kernel(AttnArgs a) {
  using SM = TQ3Smem<D, NCT>;
  constexpr int NW = SM::NW;
  constexpr int TL = SM::TL;
  constexpr int NDT = D / 32;
  constexpr int SB = tq3_sub_bytes(D);
  constexpr int NBUF = SVATTN_TQ3_NBUF;
  __shared__ __align__(16) uint8_t smem[SM::BYTES];
  uint8_t* klut = smem + SM::KLUT_OFF;
  float* cbuf = reinterpret_cast<float*>(smem + SM::CBUF_OFF);
  uint32_t* vlut = reinterpret_cast<uint32_t*>(smem + SM::VLUT_OFF);

  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; readfirstlane makes the compiler see it, so
  // tile indices and block-table reads stay scalar (no wait on vector loads)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t* scl = reinterpret_cast<uint32_t*>(smem + SM::SCL_OFF) + wave * 96;
  const int ct = wave % NCT, tl = wave / NCT;
  uint8_t* qf = smem + SM::qf_off(ct);
  const int col = lane & 31, hh = lane >> 5;
  const int c = ct * 32 + col;
  const int w = blockIdx.x;
  const Chunk ch = chunk_of(a, w);
  const int s = ch.s, h = ch.h, tlo = ch.tlo;
  const int L = ch.L, n = ch.n;
  const int R = n * a.g;
  const bool col_ok = c < R;
  const int row_i = col_ok ? c / a.g : 0;
  const int head_j = col_ok ? c - row_i * a.g : 0;
  const int ppos = L - n + row_i;

  // Block-table entries of 64 consecutive blocks from tb, one per lane: a
  // sub-tile's block is then a lane read, with no memory round trip in the
  // loop (a scalar load there waits on the counter it shares with the LDS
  // reads, draining them).  The entries are reloaded whenever a block falls
  // outside [tb, tb + 64); each wave visits its blocks in ascending order.
  const int32_t* trow = a.table + (int64_t)ch.seq * a.max_bps;
  auto tab_load = [&](int b0) { return trow[min(b0 + lane, a.max_bps - 1)]; };
  int tb = (tlo + ch.t_begin) >> 3;
  int tab = tab_load(tb);
  auto sub_of = [&](int t) {
    const int key0 = (tlo + t) * 32;
    const int blk = key0 >> 8;
    if ((unsigned)(blk - tb) >= 64u) {
      tb = blk;
      tab = tab_load(tb);
    }
    const int e = __builtin_amdgcn_readlane(tab, blk - tb);
    return a.pool + (int64_t)e * a.lay.block_bytes + ((int64_t)h * 8 + ((key0 & 255) >> 5)) * SB;
  };
  const int t_first = ch.t_begin + tl;
  const int cnt = t_first < ch.t_end ? (ch.t_end - t_first + TL - 1) / TL : 0;
  TQ3Regs<D> buf[NBUF];
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j)
    if (j < cnt) load_tq3<D>(buf[j], sub_of(t_first + j * TL), lane);

  QFrags<D> qr;
  // the 8 levels pass through LDS (wave 0's scale slice, unused until the loop)
  if (threadIdx.x == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) scl[j] = a.lev16_bits[j];  // constant indices: scalar argument reads
  }
  __syncthreads();
  {
    // key table: byte (two nibbles code | sign << 3) -> (levels, signs), one
    // copy per lane slot; value table: 6 bits of codes -> 2 levels, likewise
    const uint32_t* lv = reinterpret_cast<const uint32_t*>(smem + SM::SCL_OFF);
    // dword j of the key table is row j >> 6, half (j >> 5) & 1, slot j & 31:
    // consecutive lanes store consecutive dwords
    for (int j = threadIdx.x; j < 256 * 64; j += NW * 64) {
      const uint32_t i = j >> 6, lo = i & 15, hi = i >> 4;
      reinterpret_cast<uint32_t*>(klut)[j] =
          (j & 32) ? (((lo & 8) ? 0x3C00u : 0xBC00u) | (((hi & 8) ? 0x3C00u : 0xBC00u) << 16))
                   : (lv[lo & 7] | (lv[hi & 7] << 16));
    }
    for (int idx = threadIdx.x; idx < 64 * 32; idx += NW * 64) {
      const int e = idx >> 5;  // entry; idx & 31 is the lane slot
      vlut[idx] = lv[e & 7] | (lv[e >> 3] << 16);
    }
    const int64_t qrow = ((int64_t)(ch.qrow0 + row_i) * a.hq + h * a.gq + a.head0 + head_j) * D;
    // fp16 hi/lo pairs of q' (h1, l1) and of q'' (h2, l2) at k-step kk
    auto frags = [&](int kk, u32x4_t& h1, u32x4_t& l1, u32x4_t& h2, u32x4_t& l2) {
      h1 = l1 = h2 = l2 = u32x4_t{};
      if (!col_ok) return;
      const float* q1p = a.q + qrow + 16 * kk + 8 * hh;
      const float* q2p = a.q2 + qrow + 16 * kk + 8 * hh;
      const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(q1p);
      const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(q1p + 4);
      const f32x4_t y0 = *reinterpret_cast<const f32x4_t*>(q2p);
      const f32x4_t y1 = *reinterpret_cast<const f32x4_t*>(q2p + 4);
      // the score multiplier is applied to the scores, not to the
      // fragments: that keeps the low-order parts out of the fp16
      // subnormal range
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float xa = e < 4 ? x0[e] : x1[e - 4], xb = e < 4 ? x0[e + 1] : x1[e - 3];
        const float ya = (e < 4 ? y0[e] : y1[e - 4]) * a.q2_mul;
        const float yb = (e < 4 ? y0[e + 1] : y1[e - 3]) * a.q2_mul;
        const u32x2_t sx = split_f16_pair(xa, xb), sy = split_f16_pair(ya, yb);
        h1[e / 2] = sx[0];
        l1[e / 2] = sx[1];
        h2[e / 2] = sy[0];
        l2[e / 2] = sy[1];
      }
    };
    // query fragments of this wave's column group: k-steps tl, tl + TL, ...
    for (int kk = tl; kk < D / 16; kk += TL) {
      u32x4_t h1, l1, h2, l2;
      frags(kk, h1, l1, h2, l2);
      *reinterpret_cast<u32x4_t*>(qf + qfrag_off<D>(0, kk, lane)) = h1;
      *reinterpret_cast<u32x4_t*>(qf + qfrag_off<D>(1, kk, lane)) = h2;
      *reinterpret_cast<u32x4_t*>(qf + qfrag_off<D>(2, kk, lane)) = l1;
      *reinterpret_cast<u32x4_t*>(qf + qfrag_off<D>(3, kk, lane)) = l2;
    }
  }
  const uint32_t kslot = 0x10000u | ((uint32_t)(lane & 31) * 4);  // table base (byte 2) | slot (byte 0)
  __syncthreads();

  qr.init(qf, lane);
  ColState<D> cs;
  cs.m = NEG_INF;
  cs.l = 0.0f;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) cs.acc[dt] = f32x16_t{};

  // A wave's LDS accesses execute in order: sub-tile k reads its scales from
  // slot k & 1, and the scales of sub-tile k + 1 go to the other slot after
  // sub-tile k is processed.  Staging them before would wait for the load
  // just issued (with a two-deep ring, sub-tile k + 1's) and so expose the
  // whole memory latency once per sub-tile.  Lanes 48..63 hold copies of
  // lanes 32..47's scale words and store them to the same places, so the
  // stores need no branch.
  const int sl = lane < 48 ? lane : lane - 16;
  auto stage = [&](int k, const TQ3Regs<D>& b) { scl[(k & 1) * 48 + sl] = b.sc; };
  auto step = [&](int k, const TQ3Regs<D>& cur, const TQ3Regs<D>& next) {
    __builtin_amdgcn_wave_barrier();
    process_tq3<D, CAP>(cs, cur, qr, smem, vlut + (lane & 31), scl + (k & 1) * 48, a,
                            (tlo + t_first + k * TL) * 32, L, n, ppos, lane, kslot);
    stage(k + 1, next);
    __builtin_amdgcn_wave_barrier();
  };
  if (cnt > 0) stage(0, buf[0]);
  // the two waves of a SIMD (waves w and w + 4) start half a phase apart, so
  // that one is in its matrix-core phase while the other is in its softmax
  if (wave >= 4) __builtin_amdgcn_s_sleep(24);
  // Whole rounds of NBUF sub-tiles, then the last ones (fewer than NBUF, all
  // in flight already).  Inside a round the prefetch is unconditional: past
  // the end it reloads the last sub-tile into the ring slot that no
  // sub-tile uses any more (and its scales go to a slot nothing reads).  A
  // conditional prefetch would join two paths with different numbers of
  // loads in flight, and the compiler's wait counts then assume the worse
  // one: the wait for sub-tile k would also wait for the loads just issued.
  int i = 0;
  for (; i + NBUF <= cnt; i += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int k = i + u;
      load_tq3<D>(buf[(u + NBUF - 1) % NBUF], sub_of(t_first + min(k + NBUF - 1, cnt - 1) * TL), lane);
      step(k, buf[u], buf[(u + 1) % NBUF]);
    }
  }
#pragma unroll
  for (int u = 0; u + 1 < NBUF; ++u)
    if (i + u < cnt) step(i + u, buf[u], buf[(u + 1) % NBUF]);
  __syncthreads();  // the combine buffer overlays the tables
  combine_and_store<D, NCT, NW>(cs, cbuf, a, w, ch.k, s, h, row_i, head_j, col_ok, lane, ct, tl);
}

// ---- d = 256 on wave pairs ----------------------------------------------------------

// Half hf of a d = 256 sub-tile's bytes (key-code planes 2hf and 2hf + 1,
// value-code planes 2hf and 2hf + 1, the scales), in the d = 128 register
// layout: a wave of a pair then runs the d = 128 code on its 128 dimensions.
__device__ __forceinline__ void load_tq3_half(TQ3Regs<128>& t, const uint8_t* __restrict__ sub, int hf, int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint8_t* kp = sub + (2 * hf + j) * 1024 + lane * 16;
    const uint8_t* vp = sub + 16 * 256 + (2 * hf + j) * 768 + lane * 12;
    if constexpr (SVATTN_TQ3_NT) {
      t.kc[j] = ld_stream(kp);
      t.vc[j][0] = ld_stream_u32(vp);
      t.vc[j][1] = ld_stream_u32(vp + 4);
      t.vc[j][2] = ld_stream_u32(vp + 8);
    } else {
      t.kc[j] = *reinterpret_cast<const u32x4_t*>(kp);
      t.vc[j][0] = reinterpret_cast<const uint32_t*>(vp)[0];
      t.vc[j][1] = reinterpret_cast<const uint32_t*>(vp)[1];
      t.vc[j][2] = reinterpret_cast<const uint32_t*>(vp)[2];
    }
  }
  const uint8_t* sp = sub + 28 * 256 + (lane < 48 ? lane : lane - 16) * 4;
  if constexpr (SVATTN_TQ3_NT)
    t.sc = ld_stream_u32(sp);
  else
    t.sc = *reinterpret_cast<const uint32_t*>(sp);
}

// Shared memory of the pair kernel (eight waves: four token lanes x two
// halves of the dimensions, one 32-column group).  Below 64 KiB: the value
// table, the scale slices and each half's query fragments (q'' hi, q' lo,
// q'' lo; q' hi stays in registers); the key table in the next 64 KiB as in
// the one-wave kernels; above it one 4 KiB slot per wave for its partial
// scores.  The combine buffers (one per half) reuse the fragments and the
// key table after the loop.
struct TQ3PairSmem {
  static constexpr int VLUT_OFF = 0;
  static constexpr int SCL_OFF = 8192;
  static constexpr int FLAG_OFF = SCL_OFF + 8 * 2 * 48 * 4;  // per wave: scores ready, partner's read
  static constexpr int QF_OFF = 12288;
  static constexpr int QF_HALF = 3 * 8 * 1024;
  static constexpr int KLUT_OFF = 65536;
  static constexpr int XCH_OFF = 131072;
  static constexpr int BYTES = XCH_OFF + 8 * 4096;
  static constexpr int CBUF_OFF = QF_OFF;
  static constexpr int CBUF_HALF = CombineBuf<128, 1, 4>::FLOATS;  // floats
  static_assert(FLAG_OFF + 2 * 8 * 4 <= QF_OFF, "scale slices and flags");
  static_assert(QF_OFF + 2 * QF_HALF <= KLUT_OFF, "query fragments");
  static_assert(BYTES <= 160 * 1024, "LDS of one workgroup");
  static_assert(CBUF_OFF + 2 * CBUF_HALF * 4 <= XCH_OFF, "combine buffers");
};

// d = 256: every 32-key sub-tile is taken by a pair of waves (2p, 2p + 1,
// on two SIMDs), each holding half of the dimensions: its query fragments,
// key and value codes, key products and output accumulators are those of
// the d = 128 kernel.  The two halves' partial scores (linear in the
// products: n16 <q', c> + gamma <q'', b> over each half) meet in LDS and
// are added, half 0's first, so both waves hold the same scores, run the
// same softmax and keep the same (m, l).  The pair synchronises through two
// LDS counters per wave (scores written, partner's scores read), so pairs
// run independently and the two waves on a SIMD (pairs p and p + 2) can be
// in different phases, as in the d = 128 kernel.  Every wait is bounded.
// Two waves per SIMD fit the d = 128 register budget.
template <bool CAP>
__global__ __launch_bounds__(512) void attn_tq3_pair_kernel(AttnArgs a) {
  constexpr int D = 256, DH = 128, TL = 4;
  constexpr int SB = tq3_sub_bytes(D);
  using SM = TQ3PairSmem;
  __shared__ __align__(16) uint8_t smem[SM::BYTES];
  uint8_t* klut = smem + SM::KLUT_OFF;
  uint32_t* vlut = reinterpret_cast<uint32_t*>(smem + SM::VLUT_OFF);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tl = wave >> 1, hf = wave & 1;  // token lane (pair), half of the dimensions
  uint32_t* scl = reinterpret_cast<uint32_t*>(smem + SM::SCL_OFF) + wave * 96;
  uint8_t* qf = smem + SM::QF_OFF + hf * SM::QF_HALF;
  // the exchange slots and counters, as LDS pointers (a generic pointer
  // would make the counter reads flat loads, which wait for the sub-tile
  // loads in flight)
  typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;
  typedef __attribute__((address_space(3))) volatile uint32_t lds_flag_t;
  lds_f32x4_t* xmine = (lds_f32x4_t*)(smem + SM::XCH_OFF + wave * 4096) + lane * 4;
  const lds_f32x4_t* xother = (const lds_f32x4_t*)(smem + SM::XCH_OFF + (wave ^ 1) * 4096) + lane * 4;
  lds_flag_t* ready = (lds_flag_t*)(smem + SM::FLAG_OFF);  // [wave]: sub-tiles whose scores are out
  lds_flag_t* taken = ready + 8;  // [wave]: sub-tiles whose partner scores this wave has read
  const int col = lane & 31, hh = lane >> 5;
  const int c = col;
  const int w = blockIdx.x;
  const Chunk ch = chunk_of(a, w);
  const int s = ch.s, h = ch.h, tlo = ch.tlo;
  const int L = ch.L, n = ch.n;
  const int R = n * a.g;
  const bool col_ok = c < R;
  const int row_i = col_ok ? c / a.g : 0;
  const int head_j = col_ok ? c - row_i * a.g : 0;
  const int ppos = L - n + row_i;

  // block-table entries held one per lane, as in the one-wave kernels
  const int32_t* trow = a.table + (int64_t)ch.seq * a.max_bps;
  auto tab_load = [&](int b0) { return trow[min(b0 + lane, a.max_bps - 1)]; };
  int tb = (tlo + ch.t_begin) >> 3;
  int tab = tab_load(tb);
  auto sub_of = [&](int t) {
    const int key0 = (tlo + t) * 32;
    const int blk = key0 >> 8;
    if ((unsigned)(blk - tb) >= 64u) {
      tb = blk;
      tab = tab_load(tb);
    }
    const int e = __builtin_amdgcn_readlane(tab, blk - tb);
    return a.pool + (int64_t)e * a.lay.block_bytes + ((int64_t)h * 8 + ((key0 & 255) >> 5)) * SB;
  };
  const int t_first = ch.t_begin + tl;
  const int cnt = t_first < ch.t_end ? (ch.t_end - t_first + TL - 1) / TL : 0;
  TQ3Regs<DH> buf[2];
  if (cnt > 0) load_tq3_half(buf[0], sub_of(t_first), hf, lane);

  QFrags<DH, 1, 1> qr;  // q' hi in registers; q'' hi, q' lo, q'' lo in LDS
  if (threadIdx.x == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) scl[j] = a.lev16_bits[j];
  }
  if (threadIdx.x < 16) ready[threadIdx.x] = 0u;  // and taken[]
  __syncthreads();
  {
    const uint32_t* lv = reinterpret_cast<const uint32_t*>(smem + SM::SCL_OFF);
    for (int j = threadIdx.x; j < 256 * 64; j += 512) {
      const uint32_t i = j >> 6, lo = i & 15, hi = i >> 4;
      reinterpret_cast<uint32_t*>(klut)[j] =
          (j & 32) ? (((lo & 8) ? 0x3C00u : 0xBC00u) | (((hi & 8) ? 0x3C00u : 0xBC00u) << 16))
                   : (lv[lo & 7] | (lv[hi & 7] << 16));
    }
    for (int idx = threadIdx.x; idx < 64 * 32; idx += 512) {
      const int e = idx >> 5;
      vlut[idx] = lv[e & 7] | (lv[e >> 3] << 16);
    }
    // this half's query fragments: k-steps 8 hf .. 8 hf + 7 of the head
    const int64_t qrow = ((int64_t)(ch.qrow0 + row_i) * a.hq + h * a.gq + a.head0 + head_j) * D + DH * hf;
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk) {
      u32x4_t h1{}, l1{}, h2{}, l2{};
      if (col_ok) {
        const float* q1p = a.q + qrow + 16 * kk + 8 * hh;
        const float* q2p = a.q2 + qrow + 16 * kk + 8 * hh;
        const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(q1p);
        const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(q1p + 4);
        const f32x4_t y0 = *reinterpret_cast<const f32x4_t*>(q2p);
        const f32x4_t y1 = *reinterpret_cast<const f32x4_t*>(q2p + 4);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float xa = e < 4 ? x0[e] : x1[e - 4], xb = e < 4 ? x0[e + 1] : x1[e - 3];
          const float ya = (e < 4 ? y0[e] : y1[e - 4]) * a.q2_mul;
          const float yb = (e < 4 ? y0[e + 1] : y1[e - 3]) * a.q2_mul;
          const u32x2_t sx = split_f16_pair(xa, xb), sy = split_f16_pair(ya, yb);
          h1[e / 2] = sx[0];
          l1[e / 2] = sx[1];
          h2[e / 2] = sy[0];
          l2[e / 2] = sy[1];
        }
      }
      qr.f[0][kk] = __builtin_bit_cast(f16x8_t, h1);
      if (kk % TL == tl) {
        *reinterpret_cast<u32x4_t*>(qf + qfrag_off<DH, 1>(1, kk, lane)) = h2;
        *reinterpret_cast<u32x4_t*>(qf + qfrag_off<DH, 1>(2, kk, lane)) = l1;
        *reinterpret_cast<u32x4_t*>(qf + qfrag_off<DH, 1>(3, kk, lane)) = l2;
      }
    }
  }
  const uint32_t kslot = 0x10000u | ((uint32_t)(lane & 31) * 4);
  __syncthreads();

  qr.init(qf, lane);
  ColState<DH> cs;
  cs.m = NEG_INF;
  cs.l = 0.0f;
#pragma unroll
  for (int dt = 0; dt < DH / 32; ++dt) cs.acc[dt] = f32x16_t{};

  const int sl = lane < 48 ? lane : lane - 16;
  auto stage = [&](int k, const TQ3Regs<DH>& b) { scl[(k & 1) * 48 + sl] = b.sc; };
  // Wait (bounded) until counter f reaches v; every lane reads the same
  // word.  The LDS serves a wave's accesses in order; the empty asm keeps the
  // compiler from moving LDS accesses across the wait.
  auto wait_for = [](lds_flag_t* f, uint32_t v) {
    for (int i = 0; i < (1 << 22); ++i) {
      if (*f >= v) break;
      __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
  };
  // the partial scores out and the other half's in (sub-tile xk of the
  // pair): scores = half 0's + half 1's in both waves.  The slot is
  // rewritten only once the partner has read its previous contents.
  uint32_t xk = 0;
  auto exchange = [&](float (&p)[16]) {
    if (xk > 0) wait_for(&taken[wave ^ 1], xk);
#pragma unroll
    for (int j = 0; j < 4; ++j) xmine[j] = f32x4_t{p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]};
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the scores are in LDS before the counter moves
    ready[wave] = xk + 1;
    wait_for(&ready[wave ^ 1], xk + 1);
    f32x4_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = xother[j];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the partner may rewrite its slot
    taken[wave] = xk + 1;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) p[4 * j + e] = hf == 0 ? p[4 * j + e] + o[j][e] : o[j][e] + p[4 * j + e];
    ++xk;
  };
  auto step = [&](int k, const TQ3Regs<DH>& cur, TQ3Regs<DH>& next) {
    __builtin_amdgcn_wave_barrier();
    process_tq3<DH, CAP>(cs, cur, qr, smem, vlut + (lane & 31), scl + (k & 1) * 48, a,
                         (tlo + t_first + k * TL) * 32, L, n, ppos, lane, kslot, exchange);
    stage(k + 1, next);
    __builtin_amdgcn_wave_barrier();
  };
  if (cnt > 0) stage(0, buf[0]);
  // pairs 2 and 3 (waves 4..7, the second wave of each SIMD) start half a
  // phase after pairs 0 and 1
  if (wave >= 4) __builtin_amdgcn_s_sleep(24);
  // the ring as in the one-wave kernels: whole rounds of two, the prefetch
  // unconditional (past the end it reloads the last sub-tile), then the last
  int k = 0;
  for (; k + 2 <= cnt; k += 2) {
    load_tq3_half(buf[1], sub_of(t_first + min(k + 1, cnt - 1) * TL), hf, lane);
    step(k, buf[0], buf[1]);
    load_tq3_half(buf[0], sub_of(t_first + min(k + 2, cnt - 1) * TL), hf, lane);
    step(k + 1, buf[1], buf[0]);
  }
  if (k < cnt) step(k, buf[0], buf[1]);
  // the combine buffers overlay the fragments and tables
  __syncthreads();
  float* cbuf = reinterpret_cast<float*>(smem + SM::CBUF_OFF) + hf * SM::CBUF_HALF;
  combine_and_store<DH, 1, 4, D>(cs, cbuf, a, w, ch.k, s, h, row_i, head_j, col_ok, lane, 0, tl, DH * hf, hf == 0);
}

template <int D, int NCT>
static hipError_t launch_tq3_dn(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.n_wg), block(TQ3Cfg<D>::NW * 64);
  if (a.softcap > 0.0f)
    hipLaunchKernelGGL((attn_tq3_kernel<D, NCT, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((attn_tq3_kernel<D, NCT, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_tq3(const AttnArgs& a, int nct, hipStream_t s) {
  if (a.n_wg <= 0) return hipSuccess;
  const int d = a.lay.d;
  if (d == 64) return nct == 1 ? launch_tq3_dn<64, 1>(a, s) : launch_tq3_dn<64, 2>(a, s);
  if (d == 128) return nct == 1 ? launch_tq3_dn<128, 1>(a, s) : launch_tq3_dn<128, 2>(a, s);
  if (d == 256 && nct == 1) {
    dim3 grid(a.n_wg), block(512);
    if (a.softcap > 0.0f)
      hipLaunchKernelGGL(attn_tq3_pair_kernel<true>, grid, block, 0, s, a);
    else
      hipLaunchKernelGGL(attn_tq3_pair_kernel<false>, grid, block, 0, s, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace svattn
