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

#define NEG_INF (-__builtin_inff())

// Key (0..63) of the tile held by MFMA row m (0..31) of QK sub-tile st.
__device__ __forceinline__ int key_of_row(int st, int m) {
  return 32 * st + 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}
// Key (0..63) of score register r (0..15) of sub-tile st in half-wave hh.
__device__ __forceinline__ int key_of_reg(int st, int r, int hh) {
  return 32 * st + 16 * (r >> 3) + 8 * hh + (r & 7);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int FMT>
struct Elem;
template <>
struct Elem<0> {
  using T = float;
  static constexpr int bytes = 4;
};
template <>
struct Elem<1> {
  using T = uint16_t;
  static constexpr int bytes = 2;
};

// Per-lane state of one column of the online softmax.
template <int D>
struct ColState {
  static constexpr int NDT = D / 32;
  float m;  // running max (log2 units), same in both half-waves
  float l;  // running sum of this lane's keys
  f32x16_t acc[NDT];
};

// ---- QK and PV for the plain formats -------------------------------------------

// Query operand of one lane (column c, half hh).
template <int FMT, int D>
struct QOperand;

template <int D>
struct QOperand<1, D> {  // bf16: k-step kk holds dims 16kk + 8hh .. +8
  bf16x8_t v[D / 16];
  __device__ void load(const float* q, bool ok, int hh) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[kk][e] = (__bf16)(ok ? q[16 * kk + 8 * hh + e] : 0.0f);
    }
  }
};

template <int D>
struct QOperand<0, D> {  // fp32: k-step kk holds dim (D/2)*hh + kk
  float v[D / 2];
  __device__ void load(const float* q, bool ok, int hh) {
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) v[kk] = ok ? q[(D / 2) * hh + kk] : 0.0f;
  }
};

// S^T for sub-tile st of the tile at kt (K rows [64][D]).
template <int D>
__device__ __forceinline__ f32x16_t qk_subtile(const QOperand<1, D>& q, const uint16_t* __restrict__ kt, int st,
                                               int lane) {
  const int m = lane & 31, ha = lane >> 5;
  const uint16_t* row = kt + key_of_row(st, m) * D + 8 * ha;
  bf16x8_t kop[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) kop[kk] = *reinterpret_cast<const bf16x8_t*>(row + 16 * kk);
  f32x16_t s = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], q.v[kk], s, 0, 0, 0);
  return s;
}

template <int D>
__device__ __forceinline__ f32x16_t qk_subtile(const QOperand<0, D>& q, const float* __restrict__ kt, int st,
                                               int lane) {
  const int m = lane & 31, ha = lane >> 5;
  const float* row = kt + key_of_row(st, m) * D + (D / 2) * ha;
  f32x16_t s = {};
#pragma unroll
  for (int kk = 0; kk < D / 2; kk += 4) {
    f32x4_t k4 = *reinterpret_cast<const f32x4_t*>(row + kk);
#pragma unroll
    for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(k4[e], q.v[kk + e], s, 0, 0, 0);
  }
  return s;
}

// O^T += V^T P^T for a 64-key tile; vt = V sub-tile [D][64]; p = probabilities
// in score-register order; nvalid = keys of the tile below seq_len (64 if all).
template <int D>
__device__ __forceinline__ void pv_tile(ColState<D>& st, const uint16_t* __restrict__ vt, const float (&p)[2][16],
                                        int lane, int nvalid) {
  const int dr = lane & 31, ha = lane >> 5;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    // P = hi + lo, both bf16: the residual of a float after rounding to bf16
    // is exact in fp32, so hi + lo carries P to about 2^-17 relative, and the
    // product with the bf16 values is accumulated in fp32 by the MFMA.
    bf16x8_t phi, plo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = p[u >> 1][8 * (u & 1) + e];
      const __bf16 h = (__bf16)x;
      phi[e] = h;
      plo[e] = (__bf16)(x - (float)h);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const uint16_t* src = vt + (32 * dt + dr) * 64 + 16 * u + 8 * ha;
      u16x8_t raw = *reinterpret_cast<const u16x8_t*>(src);
      if (nvalid < 64) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (16 * u + 8 * ha + e >= nvalid) raw[e] = 0;
      }
      const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, raw);
      st.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, phi, st.acc[dt], 0, 0, 0);
      st.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, plo, st.acc[dt], 0, 0, 0);
    }
  }
}

template <int D>
__device__ __forceinline__ void pv_tile(ColState<D>& st, const float* __restrict__ vt, const float (&p)[2][16],
                                        int lane, int nvalid) {
  const int dr = lane & 31, ha = lane >> 5;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const float* rowp = vt + (32 * dt + dr) * 64;
#pragma unroll
    for (int u4 = 0; u4 < 32; u4 += 4) {
      // keys of u = u4..u4+3 for half ha: 32(u>>4) + 16((u>>3)&1) + 8ha + (u&7)
      const int kbase = 32 * (u4 >> 4) + 16 * ((u4 >> 3) & 1) + 8 * ha + (u4 & 7);
      f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(rowp + kbase);
      if (nvalid < 64) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kbase + e >= nvalid) v4[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int u = u4 + e;
        st.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(v4[e], p[u >> 4][u & 15], st.acc[dt], 0, 0, 0);
      }
    }
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

template <int FMT, int D, int NCT>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  using T = typename Elem<FMT>::T;
  constexpr int TL = 4 / NCT;  // token lanes
  constexpr int NDT = D / 32;
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
    const int tlo = klo / kTileKeys;
    const int nt = (L + kTileKeys - 1) / kTileKeys - tlo;
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
    qop.load(a.q + ((int64_t)(a.qrow0[s] + row_i) * a.hq + h * a.g + head_j) * D, col_ok, hh);

    ColState<D> cs;
    cs.m = NEG_INF;
    cs.l = 0.0f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) cs.acc[dt] = f32x16_t{};

    const int32_t* trow = a.table + (int64_t)a.seq[s] * a.max_bps;
    for (int t = t_begin + tl; t < t_end; t += TL) {
      const int key0 = (tlo + t) * kTileKeys;
      const int blk = trow[key0 >> 8];
      const uint8_t* bbase = a.pool + (int64_t)blk * a.lay.block_bytes;
      const T* kt = reinterpret_cast<const T*>(bbase + a.lay.k_off) + ((int64_t)h * 256 + (key0 & 255)) * D;
      const T* vt = reinterpret_cast<const T*>(bbase + a.lay.v_off) + ((int64_t)h * 4 + ((key0 & 255) >> 6)) * D * 64;

      float p[2][16];
      f32x16_t s0 = qk_subtile<D>(qop, kt, 0, lane);
      f32x16_t s1 = qk_subtile<D>(qop, kt, 1, lane);
      float mt = NEG_INF;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = st == 0 ? s0[r] : s1[r];
          float sc = x * a.scale;
          if (a.softcap > 0.0f) sc = a.softcap * tanhf(sc * a.inv_softcap);
          sc *= 1.4426950408889634f;  // log2(e): the softmax runs on exp2
          const int kp = key0 + key_of_reg(st, r, hh);
          const bool vis = col_ok && kp <= ppos && (a.window == 0 || ppos - kp < a.window);
          sc = vis ? sc : NEG_INF;
          p[st][r] = sc;
          mt = fmaxf(mt, sc);
        }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(cs.m, mt);
      const float m_use = m_new == NEG_INF ? 0.0f : m_new;
      const float alpha = fast_exp2(cs.m - m_use);
      float lsum = 0.0f;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = fast_exp2(p[st][r] - m_use);
          p[st][r] = e;
          lsum += e;
        }
      }
      cs.l = cs.l * alpha + lsum;
      cs.m = m_new;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) cs.acc[dt] *= alpha;
      pv_tile<D>(cs, vt, p, lane, min(64, L - key0));
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
  const int tlo = klo / kTileKeys;
  const int nt = (L + kTileKeys - 1) / kTileKeys - tlo;
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
  if (nct == 1)
    hipLaunchKernelGGL((attn_kernel<FMT, D, 1>), dim3(a.n_wg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<FMT, D, 2>), dim3(a.n_wg), dim3(256), 0, s, a);
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
