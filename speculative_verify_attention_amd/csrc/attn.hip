// attn.hip - verify attention over the paged cache on gfx950.
//
// The path: 1+k query rows per sequence (AX Engine page, "Core Technical
// Architecture & Methods": up to 4 drafts per step, checked in one forward;
// SwiftLM page, speculative-decoding passage: N+1 positions verified
// together), grouped-query heads (AX Engine page, "Supported Model Families":
// dense GQA), causal offsets for the draft rows, an optional sliding window
// and logit soft cap (same section, Gemma4; mlx-engine blog, model
// architecture section: 512-token local windows).
//
// Design for gfx950:
//  * Work unit = 64-key tile of one (sequence, kv head).  All 1+k rows of all
//    g query heads of that kv head share each K/V byte, so every stored byte
//    is read from HBM once per call.
//  * The flat list of tiles over (sequence, kv head) is cut into equal
//    contiguous ranges, one per workgroup (split-context): long and short
//    sequences in one batch cost the same per workgroup.  A range that does
//    not cover a whole (sequence, kv head) leaves a partial (m, l, acc) in the
//    workspace; the merge kernel combines them by log-sum-exp.
//  * Inside a workgroup, 4 wavefronts take tiles round-robin (token lanes)
//    and keep their own online-softmax state; at the end of a range the
//    states are combined through LDS.  With more than 32 (row, head) columns
//    the waves split into two column groups instead.
//  * Products run on MFMA 32x32 with keys as the M dimension and query
//    columns as N: S^T = K Q^T, then O^T += V^T P^T.  K rows and V^T rows
//    (V is stored token-minor per 64-token sub-tile) are loaded straight
//    into MFMA operand registers with 16-byte loads; the key order inside a
//    tile is permuted so that the score registers a lane holds are exactly
//    the P operand it feeds into the PV product (no shuffles, no LDS).
//  * Per column, the row max is reduced across the two half-waves with one
//    exchange per tile; the row sum stays per lane until the end.
#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "kernels.h"
#include "lanes.h"

// Query fragments re-read from LDS at every tile from this head size up (0:
// never), and the largest tile (registers per lane) kept in a ring of
// SVATTN_NBUF tiles; bigger tiles are loaded one at a time.
#ifndef SVATTN_Q_FROM_LDS
#define SVATTN_Q_FROM_LDS 256
#endif
#ifndef SVATTN_RING_MAX_REGS
#define SVATTN_RING_MAX_REGS 64
#endif
// Bigger tiles: one buffer refilled in halves (K, then V) instead of whole.
#ifndef SVATTN_STAGGER
#define SVATTN_STAGGER 1
#endif
// Non-temporal hint on the tile loads from this head size down (the
// measured choice: faster at d <= 128, slower at d = 256, where one tile
// buffer is refilled in halves).
#ifndef SVATTN_NT_MAX_D
#define SVATTN_NT_MAX_D 128
#endif

namespace svattn {

// ---- per-format traits ---------------------------------------------------------------
//
// A tile is NSUB sub-tiles of 32 keys.  A sub-tile's K and V occupy LK and LV
// wave-wide 1 KiB loads (lane l reads 16 bytes at 16 l), laid out so the
// registers each lane receives are exactly its MFMA operand fragments.

template <int FMT, int D>
struct Tr;
template <int D>
struct Tr<1, D> {  // bf16: v_mfma_f32_32x32x16_bf16
  using Elem = uint16_t;
  static constexpr int NSUB = 128 / D > 1 ? 128 / D : 1;
  static constexpr int LK = D / 16;  // k-steps of QK
  static constexpr int LV = D / 16;  // 2 PV k-steps x D/32 output tiles
};
template <int D>
struct Tr<0, D> {  // fp32: v_mfma_f32_32x32x2f32
  using Elem = float;
  static constexpr int NSUB = 1;
  static constexpr int LK = D / 8;  // groups of 4 QK k-steps
  static constexpr int LV = D / 8;  // 4 groups of 4 PV k-steps x D/32 output tiles
};

template <int D>
__device__ __forceinline__ u32x4_t tile_ld(const uint8_t* p) {
  if constexpr (D <= SVATTN_NT_MAX_D)
    return ld_stream(p);
  else
    return *reinterpret_cast<const u32x4_t*>(p);
}

// One tile of raw operand registers.
template <int FMT, int D>
struct TileRegs {
  using T = Tr<FMT, D>;
  u32x4_t k[T::NSUB][T::LK];
  u32x4_t v[T::NSUB][T::LV];
};

template <int FMT, int D>
__device__ __forceinline__ void load_tile(TileRegs<FMT, D>& b, const uint8_t* __restrict__ kbase,
                                          const uint8_t* __restrict__ vbase, int lane) {
  using T = Tr<FMT, D>;
  constexpr int SUB_BYTES = 32 * D * (FMT == 1 ? 2 : 4);
#pragma unroll
  for (int st = 0; st < T::NSUB; ++st) {
#pragma unroll
    for (int j = 0; j < T::LK; ++j)
      b.k[st][j] = tile_ld<D>(kbase + st * SUB_BYTES + j * 1024 + lane * 16);
#pragma unroll
    for (int j = 0; j < T::LV; ++j)
      b.v[st][j] = tile_ld<D>(vbase + st * SUB_BYTES + j * 1024 + lane * 16);
  }
}

template <int FMT, int D>
__device__ __forceinline__ void load_k(TileRegs<FMT, D>& b, const uint8_t* __restrict__ kbase, int lane) {
  using T = Tr<FMT, D>;
  constexpr int SUB_BYTES = 32 * D * (FMT == 1 ? 2 : 4);
#pragma unroll
  for (int st = 0; st < T::NSUB; ++st)
#pragma unroll
    for (int j = 0; j < T::LK; ++j)
      b.k[st][j] = tile_ld<D>(kbase + st * SUB_BYTES + j * 1024 + lane * 16);
}
template <int FMT, int D>
__device__ __forceinline__ void load_v(TileRegs<FMT, D>& b, const uint8_t* __restrict__ vbase, int lane) {
  using T = Tr<FMT, D>;
  constexpr int SUB_BYTES = 32 * D * (FMT == 1 ? 2 : 4);
#pragma unroll
  for (int st = 0; st < T::NSUB; ++st)
#pragma unroll
    for (int j = 0; j < T::LV; ++j)
      b.v[st][j] = tile_ld<D>(vbase + st * SUB_BYTES + j * 1024 + lane * 16);
}

// Query operand of one lane (column c, half-wave hh).
template <int FMT, int D>
struct QOperand;

template <int D>
struct QOperand<1, D> {
  // bf16: the fragments live in LDS, shared by the workgroup's token lanes:
  // k-step kk of lane (c, hh) = dims 16kk + 8hh .. +8 at lds[kk * 64 + lane]
  // (high part) and lds[(D/16 + kk) * 64 + lane] (low part).  The fp32 query
  // is carried as two bf16 parts, q = hi + lo to ~2^-17 relative: the
  // residual of a float after rounding to bf16 is exact in fp32, and two
  // products per k-step keep the scores as close to fp32 queries as the
  // probabilities' hi + lo split keeps the value sums.
  static constexpr int LDS_ENTRIES = 2 * (D / 16) * 64;
  const u32x4_t* lds;
  // Written by one wave per column group.
  __device__ __forceinline__ static void store(u32x4_t* dst, const float* q, bool ok, int lane) {
    const int hh = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      bf16x8_t vh{}, vl{};
      if (ok) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(q + 16 * kk + 8 * hh);
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(q + 16 * kk + 8 * hh + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = e < 4 ? a[e] : b[e - 4];
          const __bf16 h = (__bf16)x;
          vh[e] = h;
          vl[e] = (__bf16)(x - (float)h);
        }
      }
      dst[kk * 64 + lane] = __builtin_bit_cast(u32x4_t, vh);
      dst[(D / 16 + kk) * 64 + lane] = __builtin_bit_cast(u32x4_t, vl);
    }
  }
};

template <int D>
struct QOperand<0, D> {  // k-step kk holds dim (D/2) hh + kk
  float v[D / 2];
  __device__ __forceinline__ void load(const float* q, int hh) {
#pragma unroll
    for (int kk = 0; kk < D / 2; kk += 4) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(q + (D / 2) * hh + kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[kk + e] = a[e];
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) v[kk] = 0.0f;
  }
};

// S^T of sub-tile st: lane (column c, half hh) gets the scores of keys
// 8(r>>2) + 4hh + (r&3), r = 0..15.
template <int D>
__device__ __forceinline__ f32x16_t qk_sub(const QOperand<1, D>& q, const TileRegs<1, D>& b, int st) {
  const int lane = threadIdx.x & 63;
  typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4_t;
  lds_u32x4_t* ql = (lds_u32x4_t*)q.lds;
#if SVATTN_Q_FROM_LDS
  // The fragments are read from LDS at every tile: hoisted out of the loop
  // they would hold 2 x D/4 registers for the whole loop (parked in
  // accumulation registers and copied back at every use), which leaves no
  // room for a second tile in flight at d = 256.
  if constexpr (D >= SVATTN_Q_FROM_LDS) asm volatile("" : "+v"(ql));
#endif
  f32x16_t s = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const bf16x8_t kop = __builtin_bit_cast(bf16x8_t, b.k[st][kk]);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, __builtin_bit_cast(bf16x8_t, ql[kk * 64 + lane]), s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, __builtin_bit_cast(bf16x8_t, ql[(D / 16 + kk) * 64 + lane]), s,
                                                0, 0, 0);
  }
  return s;
}
template <int D>
__device__ __forceinline__ f32x16_t qk_sub(const QOperand<0, D>& q, const TileRegs<0, D>& b, int st) {
  f32x16_t s = {};
#pragma unroll
  for (int kq = 0; kq < D / 8; ++kq) {
    const f32x4_t k4 = __builtin_bit_cast(f32x4_t, b.k[st][kq]);
#pragma unroll
    for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(k4[e], q.v[4 * kq + e], s, 0, 0, 0);
  }
  return s;
}

// Zero the V fragments of keys at or beyond nvalid (only in the last tile of a
// sequence, where never-written slots may hold arbitrary bits).
template <int D>
__device__ __forceinline__ void mask_v(TileRegs<1, D>& b, int nvalid, int ha) {
#pragma unroll
  for (int st = 0; st < Tr<1, D>::NSUB; ++st)
#pragma unroll
    for (int j = 0; j < Tr<1, D>::LV; ++j) {
      const int v = j / (D / 32);
      u16x8_t x = __builtin_bit_cast(u16x8_t, b.v[st][j]);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (32 * st + 16 * v + 8 * (e >> 2) + 4 * ha + (e & 3) >= nvalid) x[e] = 0;
      b.v[st][j] = __builtin_bit_cast(u32x4_t, x);
    }
}
template <int D>
__device__ __forceinline__ void mask_v(TileRegs<0, D>& b, int nvalid, int ha) {
#pragma unroll
  for (int st = 0; st < Tr<0, D>::NSUB; ++st)
#pragma unroll
    for (int j = 0; j < Tr<0, D>::LV; ++j) {
      const int uq = j / (D / 32);
      f32x4_t x = __builtin_bit_cast(f32x4_t, b.v[st][j]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (32 * st + 8 * uq + 4 * ha + e >= nvalid) x[e] = 0.0f;
      b.v[st][j] = __builtin_bit_cast(u32x4_t, x);
    }
}

// O^T += V^T P^T for one tile; p holds the probabilities in score-register
// order.  bf16: P = hi + lo (two bf16 parts; the residual of a float after
// rounding to bf16 is exact in fp32), so the product keeps P to ~2^-17.
template <int D>
__device__ __forceinline__ void pv_tile(f32x16_t (&acc)[D / 32], const TileRegs<1, D>& b,
                                        const float (&p)[Tr<1, D>::NSUB][16]) {
#pragma unroll
  for (int st = 0; st < Tr<1, D>::NSUB; ++st)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      bf16x8_t phi, plo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = p[st][8 * v + e];
        const __bf16 h = (__bf16)x;
        phi[e] = h;
        plo[e] = (__bf16)(x - (float)h);
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, b.v[st][v * (D / 32) + dt]);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, phi, acc[dt], 0, 0, 0);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, plo, acc[dt], 0, 0, 0);
      }
    }
}
template <int D>
__device__ __forceinline__ void pv_tile(f32x16_t (&acc)[D / 32], const TileRegs<0, D>& b,
                                        const float (&p)[Tr<0, D>::NSUB][16]) {
#pragma unroll
  for (int st = 0; st < Tr<0, D>::NSUB; ++st)
#pragma unroll
    for (int uq = 0; uq < 4; ++uq)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const f32x4_t v4 = __builtin_bit_cast(f32x4_t, b.v[st][uq * (D / 32) + dt]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(v4[e], p[st][4 * uq + e], acc[dt], 0, 0, 0);
      }
}

// ---- the partial kernel ----------------------------------------------------------

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// after_qk runs once the key products no longer need b.k, after_pv once the
// value products no longer need b.v (a single-buffered loop refills them
// there).
template <int FMT, int D, bool CAP, typename AfterQK = NoHook, typename AfterPV = NoHook>
__device__ __forceinline__ void process_tile(ColState<D>& cs, TileRegs<FMT, D>& b, const QOperand<FMT, D>& q,
                                             const AttnArgs& a, int key0, int L, int n, int ppos, int lane,
                                             AfterQK after_qk = AfterQK(), AfterPV after_pv = AfterPV()) {
  constexpr int NSUB = Tr<FMT, D>::NSUB;
  constexpr int TK = 32 * NSUB;
  const int hh = lane >> 5;
  float p[NSUB][16];
#pragma unroll
  for (int st = 0; st < NSUB; ++st) {
    const f32x16_t s = qk_sub<D>(q, b, st);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[r] * a.scale;
      if constexpr (CAP) x = a.softcap * tanh_nb(x * a.inv_softcap);
      p[st][r] = x * 1.4426950408889634f;  // log2(e): the softmax runs on exp2
    }
  }
  after_qk();
  // keys every row sees need no mask: all of the tile lies at or before the
  // first row's position and inside the last row's window
  const bool full = key0 + TK <= L - n + 1 && (a.window == 0 || L - key0 <= a.window);
  if (!full) {
    if (key0 + TK > L) mask_v<D>(b, L - key0, hh);
#pragma unroll
    for (int st = 0; st < NSUB; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kp = key0 + 32 * st + 8 * (r >> 2) + 4 * hh + (r & 3);
        const bool vis = kp <= ppos && (a.window == 0 || ppos - kp < a.window);
        p[st][r] = vis ? p[st][r] : NEG_INF;
      }
  }
  softmax_update<D, NSUB>(cs, p);
  pv_tile<D>(cs.acc, b, p);
  after_pv();
}

template <int FMT, int D, int NCT, bool CAP, bool APPEND>
__global__ __launch_bounds__(256, (FMT == 1 && D <= 128) ? SVATTN_BF16_WAVES : 1) void attn_kernel(AttnArgs a) {
  constexpr int TL = 4 / NCT;  // token lanes
  constexpr int NDT = D / 32;
  constexpr int TK = 32 * Tr<FMT, D>::NSUB;
  constexpr int E = FMT == 1 ? 2 : 4;
  // registers per tile buffer decide how many tiles are kept in flight
  constexpr int TILE_REGS = Tr<FMT, D>::NSUB * (Tr<FMT, D>::LK + Tr<FMT, D>::LV) * 4;
  constexpr int NBUF = TILE_REGS <= SVATTN_RING_MAX_REGS ? SVATTN_NBUF : 1;
  __shared__ float cbuf[CombineBuf<D, NCT>::FLOATS];
  __shared__ u32x4_t qlds[FMT == 1 ? NCT * QOperand<1, D>::LDS_ENTRIES : 1];

  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; readfirstlane makes the compiler see it, so
  // tile indices and block-table reads stay scalar (no wait on vector loads)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ct = wave % NCT, tl = wave / NCT;
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
  const int ppos = L - n + row_i;  // position of this column's query row

  // The table is read through the constant address space: scalar loads
  // even in the fused-append variant, whose pool stores would otherwise make
  // the compiler turn every table read into a vector load (and a wait on
  // the tile loads in flight).  Nothing writes the table during a launch.
  typedef __attribute__((address_space(4))) const int32_t cint32_t;
  cint32_t* trow = (cint32_t*)(a.table + (int64_t)ch.seq * a.max_bps);
  const int64_t head_off = (int64_t)h * 256 * D * E;
  auto block_of = [&](int key) { return trow[key >> 8]; };
  auto bases = [&](int t, const uint8_t*& kb, const uint8_t*& vb) {
    const int key0 = (tlo + t) * TK;
    const uint8_t* blk = a.pool + (int64_t)block_of(key0) * a.lay.block_bytes + head_off + (key0 & 255) * D * E;
    kb = blk + a.lay.k_off;
    vb = blk + a.lay.v_off;
  };
  if constexpr (APPEND) {
    // Fused append: write the verified rows of kv head h that fall in this
    // chunk's keys into the pool, then make them visible to the whole
    // workgroup before any tile load; every row lies in exactly one chunk of
    // the pair.  One thread per 8 consecutive dimensions of a row (at most
    // 8 rows x 32 groups = 256 items): one 16-byte load round trip, then
    // fire-and-forget stores.  Blocks the append pops are in the table
    // already (the host updates it before this launch).
    using T = typename Tr<FMT, D>::Elem;
    constexpr int G = 8;
    static_assert(8 * (D / G) <= 256, "one item per thread");
    const int lo = max((tlo + ch.t_begin) * TK, L - n), hi = min((tlo + ch.t_end) * TK, L);
    if (lo < hi) {
      const int b_lo = block_of(lo), b_hi = block_of(hi - 1);  // the rows span at most two blocks
      const int item = threadIdx.x;
      if (item < (hi - lo) * (D / G)) {
        const int p = lo + item / (D / G), d0 = (item % (D / G)) * G;
        const int64_t src = ((int64_t)(ch.qrow0 + p - (L - n)) * a.lay.hkv + h) * D + d0;
        T kx[G], vx[G];
        const u32x4_t* ks = reinterpret_cast<const u32x4_t*>(static_cast<const T*>(a.new_k) + src);
        const u32x4_t* vs = reinterpret_cast<const u32x4_t*>(static_cast<const T*>(a.new_v) + src);
#pragma unroll
        for (int j = 0; j < (int)(G * sizeof(T) / 16); ++j) {
          *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint8_t*>(kx) + 16 * j) = ks[j];
          *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint8_t*>(vx) + 16 * j) = vs[j];
        }
        uint8_t* blk = const_cast<uint8_t*>(a.pool) + (int64_t)((p >> 8) == (lo >> 8) ? b_lo : b_hi) * a.lay.block_bytes;
        T* kd = reinterpret_cast<T*>(blk + a.lay.k_off) + (int64_t)h * 256 * D;
        T* vd = reinterpret_cast<T*>(blk + a.lay.v_off) + (int64_t)h * 256 * D;
#pragma unroll
        for (int e = 0; e < G; ++e) {
          kd[plain_k_index(FMT, D, p & 255, d0 + e)] = kx[e];
          vd[plain_v_index(FMT, D, p & 255, d0 + e)] = vx[e];
        }
      }
      __threadfence_block();
      __syncthreads();
    }
  }
  const int t_first = ch.t_begin + tl;
  const int cnt = t_first < ch.t_end ? (ch.t_end - t_first + TL - 1) / TL : 0;

  // First tiles' loads go out before anything else waits on memory.
  // NBUF-deep register ring: tiles i+1 .. i+NBUF-1 are in flight while tile i
  // is computed; the loop is unrolled NBUF times so buffer indices are
  // compile-time constants.
  TileRegs<FMT, D> buf[NBUF];
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j) {
    if (j < cnt) {
      const uint8_t *kb, *vb;
      bases(t_first + j * TL, kb, vb);
      load_tile<FMT, D>(buf[j], kb, vb, lane);
    }
  }

  const float* qsrc = a.q + ((int64_t)(ch.qrow0 + row_i) * a.hq + h * a.gq + a.head0 + head_j) * D;
  QOperand<FMT, D> qop;
  if constexpr (FMT == 1) {
    if (tl == 0) QOperand<1, D>::store(qlds + ct * QOperand<1, D>::LDS_ENTRIES, qsrc, col_ok, lane);
    __syncthreads();
    qop.lds = qlds + ct * QOperand<1, D>::LDS_ENTRIES;
  } else {
    if (col_ok)
      qop.load(qsrc, hh);
    else
      qop.zero();
  }

  ColState<D> cs;
  cs.m = NEG_INF;
  cs.l = 0.0f;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) cs.acc[dt] = f32x16_t{};

  // Whole rounds of NBUF tiles, then the last tiles (fewer than NBUF, all in
  // flight already).  Inside a round the prefetch is unconditional: past the
  // end it reloads the last tile into the ring slot that no tile uses any
  // more.  A conditional prefetch would join two paths with different
  // numbers of loads in flight, and the compiler's wait counts then assume
  // the worse one: the wait for tile k would also wait for the tile just
  // requested.
  if constexpr (NBUF == 1 && FMT == 1 && SVATTN_STAGGER) {
    // One tile buffer, refilled in halves: the next tile's K is requested as
    // soon as this tile's key products are issued, its V once the value
    // products are, so each half has the other half's compute to arrive
    // (past the end the last tile is reloaded, unused).
    if (cnt > 0) {
      const uint8_t *kb, *vb;
      bases(t_first, kb, vb);
      load_tile<FMT, D>(buf[0], kb, vb, lane);
    }
    for (int k = 0; k < cnt; ++k) {
      const uint8_t *kb, *vb;
      bases(t_first + min(k + 1, cnt - 1) * TL, kb, vb);
      process_tile<FMT, D, CAP>(cs, buf[0], qop, a, (tlo + t_first + k * TL) * TK, L, n, ppos, lane,
                                [&] { load_k<FMT, D>(buf[0], kb, lane); }, [&] { load_v<FMT, D>(buf[0], vb, lane); });
    }
  } else {
    int i = 0;
    for (; i + NBUF <= cnt; i += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int k = i + u;
        const uint8_t *kb, *vb;
        bases(t_first + min(k + NBUF - 1, cnt - 1) * TL, kb, vb);
        load_tile<FMT, D>(buf[(u + NBUF - 1) % NBUF], kb, vb, lane);
        process_tile<FMT, D, CAP>(cs, buf[u], qop, a, (tlo + t_first + k * TL) * TK, L, n, ppos, lane);
      }
    }
#pragma unroll
    for (int u = 0; u + 1 < NBUF; ++u)
      if (i + u < cnt)
        process_tile<FMT, D, CAP>(cs, buf[u], qop, a, (tlo + t_first + (i + u) * TL) * TK, L, n, ppos, lane);
  }

  combine_and_store<D, NCT>(cs, cbuf, a, w, ch.k, s, h, row_i, head_j, col_ok, lane, ct, tl);
}

// ---- merge of split partials -------------------------------------------------------

// One wavefront per (sequence, kv head, query column).  Pairs that a single
// workgroup covered whole were finished by the partial kernel and are
// skipped.  The partials' maxima and sums are reduced across the wave; each
// lane then accumulates D/64 output dimensions over the partials.
template <int D, bool ROT>
__global__ __launch_bounds__(64) void merge_kernel(AttnArgs a) {
  constexpr int EL = D / 64;
  const int hkv = a.lay.hkv;
  const int rmax = a.rpad;
  const int pair = blockIdx.x / rmax, c = blockIdx.x - pair * rmax;
  const int s = pair / hkv, h = pair - s * hkv;
  // the sequence's fields, read together (one round trip) before any branch
  const int n = a.nrows[s], k = a.ksplit[s], wb = a.wg_base[s], q0 = a.qrow0[s];
  const int R = n * a.g;
  if (c >= R || (k == 1 && !a.force_partial)) return;
  const int w0 = wb + h * k;  // the pair's chunks are workgroups w0 .. w0+k-1
  const int lane = threadIdx.x;
  const float* base = a.part + (int64_t)w0 * a.slot_stride;
  // One memory round trip for k <= KB: lane j holds chunk j's (m, l), and
  // the first KB chunks' accumulator parts are loaded beside them (they do
  // not depend on the maximum).  d = 256 (few merge waves, up to 32 chunks
  // a pair): 32; d <= 128, whose merges run many more waves: 8, so that the
  // registers stay few (with 32 the dense and mixed workloads' merges took
  // 1.5-2x as long).
  constexpr int KB = D > 128 ? 32 : 8;
  float mj = NEG_INF, lj = 0.0f;
  if (lane < k) {
    mj = base[(int64_t)lane * a.slot_stride + c];
    lj = base[(int64_t)lane * a.slot_stride + a.rpad + c];
  }
  float accj[KB][EL];
#pragma unroll
  for (int j = 0; j < KB; ++j) {
    if (j < k) {
      const float* src = base + (int64_t)j * a.slot_stride + 2 * a.rpad + (int64_t)c * D + lane * EL;
#pragma unroll
      for (int e = 0; e < EL; ++e) accj[j][e] = src[e];
    }
  }
  const float m_own = mj;  // chunk `lane`'s own maximum, read back by shuffles below
  // more than 64 chunks: each lane folds chunks lane + 64, lane + 128, ...
  // into its (m, l) online
  for (int j = lane + 64; j < k; j += 64) {
    const float* slot = base + (int64_t)j * a.slot_stride;
    const float m2 = slot[c], l2 = slot[a.rpad + c];
    const float mn = fmaxf(mj, m2);
    if (mn != NEG_INF) {
      lj = lj * fast_exp2(mj - mn) + l2 * fast_exp2(m2 - mn);
      mj = mn;
    }
  }
  float M = mj;
  M = fmaxf(M, lane_xor<32>(M));
  M = fmaxf(M, lane_xor<16>(M));
  M = fmaxf(M, lane_xor<8>(M));
  M = fmaxf(M, lane_xor<4>(M));
  M = fmaxf(M, lane_xor<2>(M));
  M = fmaxf(M, lane_xor<1>(M));
  const float mu = M == NEG_INF ? 0.0f : M;
  const float lsum = lanes_sum(lj * fast_exp2(mj - mu));
  float acc[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int j = 0; j < KB; ++j) {
    if (j < k) {
      const float f = fast_exp2(lane_value(m_own, j) - mu);
#pragma unroll
      for (int e = 0; e < EL; ++e) acc[e] += accj[j][e] * f;
    }
  }
  // the other chunks KB at a time: a batch's loads are issued together (one
  // round trip per batch, not per chunk), then folded in chunk order
  for (int j0 = KB; j0 < k; j0 += KB) {
    float xj[KB][EL], mx[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int j = j0 + u;
      if (j < k) {
        const float* slot = base + (int64_t)j * a.slot_stride;
        mx[u] = j < 64 ? lane_value(m_own, j) : slot[c];
        const float* src = slot + 2 * a.rpad + (int64_t)c * D + lane * EL;
#pragma unroll
        for (int e = 0; e < EL; ++e) xj[u][e] = src[e];
      }
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (j0 + u < k) {
        const float f = fast_exp2(mx[u] - mu);
#pragma unroll
        for (int e = 0; e < EL; ++e) acc[e] += xj[u][e] * f;
      }
    }
  }
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int e = 0; e < EL; ++e) acc[e] *= inv;
  if constexpr (ROT) {
    // o = Pi^T o' = D H o' / sqrt(d): Walsh-Hadamard butterflies over the
    // wave (lane owns dims lane*EL ..), then the signs and the scale
#pragma unroll
    for (int hs = 1; hs < EL; hs <<= 1)
#pragma unroll
      for (int e = 0; e < EL; ++e)
        if (!(e & hs)) {
          const float x = acc[e], y = acc[e + hs];
          acc[e] = x + y;
          acc[e + hs] = x - y;
        }
    wht_lanes(acc, lane);
    // 1/sqrt(d) of the rotation and 1/sqrt(d) of the value reconstruction
    // (the partial kernel accumulates n16 * c16[code] without it)
    constexpr float inv_d = 1.0f / D;
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[e] *= (a.signs[lane * EL + e] < 0 ? -inv_d : inv_d);
  }
  const int row_i = c / a.g, head_j = c - row_i * a.g;
  float* o = a.out + ((int64_t)(q0 + row_i) * a.hq + h * a.gq + a.head0 + head_j) * D + lane * EL;
#pragma unroll
  for (int e = 0; e < EL; ++e) o[e] = acc[e];
}

// ---- launchers ----------------------------------------------------------------------

template <int FMT, int D, bool APPEND>
static hipError_t launch_attn_fda(const AttnArgs& a, int nct, hipStream_t s) {
  const bool cap = a.softcap > 0.0f;
  if (nct == 1 && !cap)
    hipLaunchKernelGGL((attn_kernel<FMT, D, 1, false, APPEND>), dim3(a.n_wg), dim3(256), 0, s, a);
  else if (nct == 1)
    hipLaunchKernelGGL((attn_kernel<FMT, D, 1, true, APPEND>), dim3(a.n_wg), dim3(256), 0, s, a);
  else if (!cap)
    hipLaunchKernelGGL((attn_kernel<FMT, D, 2, false, APPEND>), dim3(a.n_wg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<FMT, D, 2, true, APPEND>), dim3(a.n_wg), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int FMT, int D>
static hipError_t launch_attn_fd(const AttnArgs& a, int nct, hipStream_t s) {
  return a.new_k ? launch_attn_fda<FMT, D, true>(a, nct, s) : launch_attn_fda<FMT, D, false>(a, nct, s);
}

hipError_t launch_attn(const AttnArgs& a, int nct, hipStream_t s) {
  if (a.n_wg <= 0) return hipSuccess;
  if (nct != 1 && nct != 2) return hipErrorInvalidValue;
  const int fmt = a.lay.fmt, d = a.lay.d;
  if (fmt == 0) {
    if (d == 64) return launch_attn_fd<0, 64>(a, nct, s);
    if (d == 128) return launch_attn_fd<0, 128>(a, nct, s);
    if (d == 256) return launch_attn_fd<0, 256>(a, nct, s);
  } else if (fmt == 1) {
    if (d == 64) return launch_attn_fd<1, 64>(a, nct, s);
    if (d == 128) return launch_attn_fd<1, 128>(a, nct, s);
    if (d == 256) return launch_attn_fd<1, 256>(a, nct, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const AttnArgs& a, int nct, hipStream_t s) {
  (void)nct;
  const int blocks = a.n_seqs * a.lay.hkv * a.rpad;
  if (blocks <= 0) return hipSuccess;
  const int d = a.lay.d;
  const bool rot = a.lay.fmt == 2;
  dim3 grid(blocks), block(64);
  if (d == 64 && rot)
    hipLaunchKernelGGL((merge_kernel<64, true>), grid, block, 0, s, a);
  else if (d == 64)
    hipLaunchKernelGGL((merge_kernel<64, false>), grid, block, 0, s, a);
  else if (d == 128 && rot)
    hipLaunchKernelGGL((merge_kernel<128, true>), grid, block, 0, s, a);
  else if (d == 128)
    hipLaunchKernelGGL((merge_kernel<128, false>), grid, block, 0, s, a);
  else if (d == 256 && rot)
    hipLaunchKernelGGL((merge_kernel<256, true>), grid, block, 0, s, a);
  else if (d == 256)
    hipLaunchKernelGGL((merge_kernel<256, false>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}


}  // namespace svattn
