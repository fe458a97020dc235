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

#include "kernels.h"

namespace svattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define NEG_INF (-__builtin_inff())

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh without branches, for the soft cap: an odd Taylor polynomial below
// |x| = 0.55 (truncation below 2e-7 relative there) and 1 - 2 / (e^{2|x|} + 1)
// above, where the subtraction loses no more than a few ulp.
__device__ __forceinline__ float tanh_nb(float x) {
  const float ax = fabsf(x);
  const float x2 = x * x;
  float p = 929569.0f / 638512875.0f;
  p = fmaf(p, x2, -21844.0f / 6081075.0f);
  p = fmaf(p, x2, 1382.0f / 155925.0f);
  p = fmaf(p, x2, -62.0f / 2835.0f);
  p = fmaf(p, x2, 17.0f / 315.0f);
  p = fmaf(p, x2, -2.0f / 15.0f);
  p = fmaf(p, x2, 1.0f / 3.0f);
  const float small = fmaf(-x * x2, p, x);
  const float e = fast_exp2(ax * 2.8853900817779268f);  // e^{2|x|}
  const float big = copysignf(1.0f - 2.0f / (e + 1.0f), x);
  return ax < 0.55f ? small : big;
}

// ---- per-format traits ---------------------------------------------------------------
//
// A tile is NSUB sub-tiles of 32 keys.  A sub-tile's K and V occupy LK and LV
// wave-wide 1 KiB loads (lane l reads 16 bytes at 16 l), laid out so the
// registers each lane receives are exactly its MFMA operand fragments.

template <int FMT, int D>
struct Tr;
template <int D>
struct Tr<1, D> {  // bf16: v_mfma_f32_32x32x16_bf16
  static constexpr int NSUB = 128 / D > 1 ? 128 / D : 1;
  static constexpr int LK = D / 16;  // k-steps of QK
  static constexpr int LV = D / 16;  // 2 PV k-steps x D/32 output tiles
};
template <int D>
struct Tr<0, D> {  // fp32: v_mfma_f32_32x32x2f32
  static constexpr int NSUB = 1;
  static constexpr int LK = D / 8;  // groups of 4 QK k-steps
  static constexpr int LV = D / 8;  // 4 groups of 4 PV k-steps x D/32 output tiles
};

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
      b.k[st][j] = *reinterpret_cast<const u32x4_t*>(kbase + st * SUB_BYTES + j * 1024 + lane * 16);
#pragma unroll
    for (int j = 0; j < T::LV; ++j)
      b.v[st][j] = *reinterpret_cast<const u32x4_t*>(vbase + st * SUB_BYTES + j * 1024 + lane * 16);
  }
}

// Query operand of one lane (column c, half-wave hh).
template <int FMT, int D>
struct QOperand;

template <int D>
struct QOperand<1, D> {  // k-step kk holds dims 16kk + 8hh .. +8
  bf16x8_t v[D / 16];
  __device__ __forceinline__ void load(const float* q, int hh) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(q + 16 * kk + 8 * hh);
      const f32x4_t b = *reinterpret_cast<const f32x4_t*>(q + 16 * kk + 8 * hh + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[kk][e] = (__bf16)a[e];
        v[kk][4 + e] = (__bf16)b[e];
      }
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) v[kk] = bf16x8_t{};
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
  f32x16_t s = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b.k[st][kk]), q.v[kk], s, 0, 0, 0);
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

__device__ __forceinline__ int find_seq(const int32_t* base, int n, int f) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (base[mid] <= f)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Online-softmax state of one lane: column c's running reference max m (log2
// units, equal in both half-waves), this lane's partial sum l, and its part
// of the column's O^T accumulator.
template <int D>
struct ColState {
  float m, l;
  f32x16_t acc[D / 32];
};

template <int FMT, int D, bool CAP>
__device__ __forceinline__ void process_tile(ColState<D>& cs, TileRegs<FMT, D>& b, const QOperand<FMT, D>& q,
                                             const AttnArgs& a, int key0, int L, int n, int ppos, int lane) {
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
  float mt = NEG_INF;
#pragma unroll
  for (int st = 0; st < NSUB; ++st)
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, p[st][r]);
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  // move the reference only when the tile max exceeds it by more than 2^8,
  // so probabilities stay below 256 and rescales are rare
  const bool up = mt > cs.m + 8.0f;
  if (__builtin_amdgcn_ballot_w64(up)) {
    // lanes that move: alpha = 2^(m_old - m_new), 0 when nothing was seen yet;
    // lanes that stay keep alpha = 1 (their m may still be -inf)
    const float alpha = up ? fast_exp2(cs.m - mt) : 1.0f;
    cs.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) cs.acc[dt] *= alpha;
    cs.m = up ? mt : cs.m;
  }
  const float m_use = cs.m == NEG_INF ? 0.0f : cs.m;
  float lsum = 0.0f;
#pragma unroll
  for (int st = 0; st < NSUB; ++st)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(p[st][r] - m_use);
      p[st][r] = e;
      lsum += e;
    }
  cs.l += lsum;
  pv_tile<D>(cs.acc, b, p);
}

template <int FMT, int D, int NCT, bool CAP>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int TL = 4 / NCT;  // token lanes
  constexpr int NDT = D / 32;
  constexpr int TK = 32 * Tr<FMT, D>::NSUB;
  constexpr int E = FMT == 1 ? 2 : 4;
  constexpr bool DB = Tr<FMT, D>::NSUB * (Tr<FMT, D>::LK + Tr<FMT, D>::LV) * 4 <= 64;  // double-buffer
  constexpr int CSTRIDE = D * 32 + 64;  // floats per combine slot
  __shared__ float cbuf[NCT * (TL / 2) * CSTRIDE];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ct = wave % NCT, tl = wave / NCT;
  const int col = lane & 31, hh = lane >> 5;
  const int c = ct * 32 + col;
  const int w = blockIdx.x;
  const int hkv = a.lay.hkv;
  int f = w * a.tiles_per_wg;
  const int fend = min(f + a.tiles_per_wg, a.total_tiles);

  while (f < fend) {
    const int s = find_seq(a.tile_base, a.n_seqs, f);
    const int L = a.len[s], n = a.nrows[s];
    const int klo = a.window > 0 ? max(0, L - n - a.window + 1) : 0;
    const int tlo = klo / TK;
    const int nt = (L + TK - 1) / TK - tlo;
    const int rel = f - a.tile_base[s];
    const int h = rel / nt;
    const int pair_first = a.tile_base[s] + h * nt;
    const int seg_end = min(fend, pair_first + nt);
    const int t_begin = f - pair_first, t_end = seg_end - pair_first;
    const int R = n * a.g;
    const bool col_ok = c < R;
    const int row_i = col_ok ? c / a.g : 0;
    const int head_j = col_ok ? c - row_i * a.g : 0;
    const int ppos = L - n + row_i;  // position of this column's query row

    QOperand<FMT, D> qop;
    if (col_ok)
      qop.load(a.q + ((int64_t)(a.qrow0[s] + row_i) * a.hq + h * a.g + head_j) * D, hh);
    else
      qop.zero();

    ColState<D> cs;
    cs.m = NEG_INF;
    cs.l = 0.0f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) cs.acc[dt] = f32x16_t{};

    const int32_t* trow = a.table + (int64_t)a.seq[s] * a.max_bps;
    const int64_t head_off = (int64_t)h * 256 * D * E;
    auto bases = [&](int t, const uint8_t*& kb, const uint8_t*& vb) {
      const int key0 = (tlo + t) * TK;
      const uint8_t* blk = a.pool + (int64_t)trow[key0 >> 8] * a.lay.block_bytes + head_off + (key0 & 255) * D * E;
      kb = blk + a.lay.k_off;
      vb = blk + a.lay.v_off;
    };
    const int cnt = t_begin + tl < t_end ? (t_end - t_begin - tl + TL - 1) / TL : 0;
    TileRegs<FMT, D> b0;
    if constexpr (DB) {
      TileRegs<FMT, D> b1;
      const uint8_t *kb, *vb;
      if (cnt > 0) {
        bases(t_begin + tl, kb, vb);
        load_tile<FMT, D>(b0, kb, vb, lane);
      }
      for (int i = 0; i < cnt; i += 2) {
        const int t0 = t_begin + tl + i * TL;
        if (i + 1 < cnt) {
          bases(t0 + TL, kb, vb);
          load_tile<FMT, D>(b1, kb, vb, lane);
        }
        process_tile<FMT, D, CAP>(cs, b0, qop, a, (tlo + t0) * TK, L, n, ppos, lane);
        if (i + 1 < cnt) {
          if (i + 2 < cnt) {
            bases(t0 + 2 * TL, kb, vb);
            load_tile<FMT, D>(b0, kb, vb, lane);
          }
          process_tile<FMT, D, CAP>(cs, b1, qop, a, (tlo + t0 + TL) * TK, L, n, ppos, lane);
        }
      }
    } else {
      for (int i = 0; i < cnt; ++i) {
        const int t0 = t_begin + tl + i * TL;
        const uint8_t *kb, *vb;
        bases(t0, kb, vb);
        load_tile<FMT, D>(b0, kb, vb, lane);
        process_tile<FMT, D, CAP>(cs, b0, qop, a, (tlo + t0) * TK, L, n, ppos, lane);
      }
    }

    // ---- combine the token lanes of each column group through LDS ----
    cs.l += __shfl_xor(cs.l, 32);
#pragma unroll
    for (int half = TL / 2; half >= 1; half >>= 1) {
      if (tl >= half && tl < 2 * half) {
        float* slot = cbuf + (ct * (TL / 2) + (tl - half)) * CSTRIDE;
        if (hh == 0) {
          slot[col] = cs.m;
          slot[32 + col] = cs.l;
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) slot[64 + (dt * 16 + r) * 64 + lane] = cs.acc[dt][r];
      }
      __syncthreads();
      if (tl < half) {
        const float* slot = cbuf + (ct * (TL / 2) + tl) * CSTRIDE;
        const float mp = slot[col], lp = slot[32 + col];
        const float mm = fmaxf(cs.m, mp);
        const float mu = mm == NEG_INF ? 0.0f : mm;
        const float fs = fast_exp2(cs.m - mu), fp = fast_exp2(mp - mu);
        cs.l = cs.l * fs + lp * fp;
        cs.m = mm;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) cs.acc[dt][r] = cs.acc[dt][r] * fs + slot[64 + (dt * 16 + r) * 64 + lane] * fp;
      }
      __syncthreads();
    }

    if (tl == 0 && col_ok) {
      const int wg_lo = pair_first / a.tiles_per_wg;
      const int wg_hi = (pair_first + nt - 1) / a.tiles_per_wg;
      if (wg_lo == wg_hi && !a.force_partial) {
        const float inv = 1.0f / cs.l;
        float* o = a.out + ((int64_t)(a.qrow0[s] + row_i) * a.hq + h * a.g + head_j) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x4_t v = {cs.acc[dt][4 * j] * inv, cs.acc[dt][4 * j + 1] * inv, cs.acc[dt][4 * j + 2] * inv,
                         cs.acc[dt][4 * j + 3] * inv};
            *reinterpret_cast<f32x4_t*>(o + 32 * dt + 8 * j + 4 * hh) = v;
          }
      } else {
        const int pair = s * hkv + h;
        float* slot = a.part + (int64_t)(w + pair) * a.slot_stride;
        if (hh == 0) {
          slot[c] = cs.m;
          slot[a.rpad + c] = cs.l;
        }
        float* acc = slot + 2 * a.rpad + (int64_t)c * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x4_t v = {cs.acc[dt][4 * j], cs.acc[dt][4 * j + 1], cs.acc[dt][4 * j + 2], cs.acc[dt][4 * j + 3]};
            *reinterpret_cast<f32x4_t*>(acc + 32 * dt + 8 * j + 4 * hh) = v;
          }
      }
    }
    f = seg_end;
  }
}

// ---- merge of split partials -------------------------------------------------------

// One workgroup per (sequence, kv head).  Pairs that one workgroup covered
// whole were finished by the partial kernel and are skipped.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
  const int hkv = a.lay.hkv;
  const int pair = blockIdx.x;
  const int s = pair / hkv, h = pair - s * hkv;
  const int L = a.len[s], n = a.nrows[s];
  const int klo = a.window > 0 ? max(0, L - n - a.window + 1) : 0;
  const int tlo = klo / a.tile_keys;
  const int nt = (L + a.tile_keys - 1) / a.tile_keys - tlo;
  const int pair_first = a.tile_base[s] + h * nt;
  const int wg_lo = pair_first / a.tiles_per_wg;
  const int wg_hi = (pair_first + nt - 1) / a.tiles_per_wg;
  if (wg_lo == wg_hi && !a.force_partial) return;
  const int R = n * a.g;
  for (int idx = threadIdx.x; idx < R * (D / 4); idx += 256) {
    const int c = idx / (D / 4), d4 = idx - c * (D / 4);
    float M = NEG_INF;
    for (int w = wg_lo; w <= wg_hi; ++w) M = fmaxf(M, a.part[(int64_t)(w + pair) * a.slot_stride + c]);
    const float mu = M == NEG_INF ? 0.0f : M;
    float lsum = 0.0f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int w = wg_lo; w <= wg_hi; ++w) {
      const float* slot = a.part + (int64_t)(w + pair) * a.slot_stride;
      const float f = fast_exp2(slot[c] - mu);
      lsum += slot[a.rpad + c] * f;
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(slot + 2 * a.rpad + (int64_t)c * D + 4 * d4);
      acc += v * f;
    }
    const float inv = 1.0f / lsum;
    const int row_i = c / a.g, head_j = c - row_i * a.g;
    float* o = a.out + ((int64_t)(a.qrow0[s] + row_i) * a.hq + h * a.g + head_j) * D + 4 * d4;
    *reinterpret_cast<f32x4_t*>(o) = acc * inv;
  }
}

// ---- launchers ----------------------------------------------------------------------

template <int FMT, int D>
static hipError_t launch_attn_fd(const AttnArgs& a, int nct, hipStream_t s) {
  const bool cap = a.softcap > 0.0f;
  if (nct == 1 && !cap)
    hipLaunchKernelGGL((attn_kernel<FMT, D, 1, false>), dim3(a.n_wg), dim3(256), 0, s, a);
  else if (nct == 1)
    hipLaunchKernelGGL((attn_kernel<FMT, D, 1, true>), dim3(a.n_wg), dim3(256), 0, s, a);
  else if (!cap)
    hipLaunchKernelGGL((attn_kernel<FMT, D, 2, false>), dim3(a.n_wg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<FMT, D, 2, true>), dim3(a.n_wg), dim3(256), 0, s, a);
  return hipGetLastError();
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
  const int pairs = a.n_seqs * a.lay.hkv;
  if (pairs <= 0) return hipSuccess;
  const int d = a.lay.d;
  if (d == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(pairs), dim3(256), 0, s, a);
  else if (d == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(pairs), dim3(256), 0, s, a);
  else if (d == 256)
    hipLaunchKernelGGL(merge_kernel<256>, dim3(pairs), dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_qprep(const QPrepArgs& a, hipStream_t s) {
  (void)a;
  (void)s;
  return hipErrorNotSupported;
}

}  // namespace svattn
