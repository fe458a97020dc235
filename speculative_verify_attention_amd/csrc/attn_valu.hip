// attn_valu.hip - the verify-attention partial kernel with both products on
// the vector ALUs instead of the matrix cores, for bf16 caches at d = 64 and
// 128.  It exists to measure the choice between the two units at the verify
// step's skinny shapes (1 + k rows x a GQA group of query columns per kv
// head); the matrix-core kernel in attn.hip is the product path.
//
// Same pool layout, chunking, partial slots and merge as the matrix-core
// kernel, and the same arithmetic: the stored bf16 keys and values times
// the fp32 queries and probabilities carried as two bf16 parts (hi + lo),
// accumulated in fp32, here by v_dot2c_f32_bf16 (two products per lane and
// instruction) instead of MFMA.  At most 20 query columns per kv head (the
// planner splits wider groups into head slices).
//
// One wave takes two 32-key sub-tiles (64 keys) per iteration:
//  * Scores, one key per lane.  The K loads arrive in the matrix-core
//    operand order (lane 32h + m holds dimensions 16j + 8h .. +7 of key m);
//    one lane swap between the halves of the two sub-tiles' registers leaves
//    every lane with all dimensions of one key, so a column's query parts
//    are the same for the whole wave: the workgroup splits its columns'
//    queries into bf16 parts in LDS once, and every wave reads them as
//    broadcasts (one 16-byte read per four dot products).  Scalar loads of
//    the parts were tried first: a column's parts (512 bytes at d = 128) do
//    not stay in the scalar cache, and each load waited for an L2 round
//    trip.  The column loop runs over the call's columns only (no padding
//    to a tile width).
//  * Per column: softmax across the wave (max by DPP and lane swaps, the
//    lazy reference max of the matrix-core kernel), probabilities split into
//    bf16 parts and packed into key pairs through LDS, then the value
//    products with one output dimension per lane: the V loads give lane
//    32h + r dimension 32dt + r of key pairs of half h, so each lane
//    accumulates its d/32 dimensions over half of the keys (halves added at
//    the end of the chunk).  Per-column state (scores, partial sums,
//    reference max, accumulators) lives in LDS, so registers hold only the
//    two sub-tiles in use and the two in flight.
#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "kernels.h"

namespace svattn {

namespace {

constexpr int kValuCols = kValuMaxCols;  // query columns one workgroup holds

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo * b.lo + a.hi * b.hi + c (bf16 pairs, fp32 accumulate)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Value of lane l ^ 16 (one lane swap between the 16-lane rows of each half).
__device__ __forceinline__ float xor16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}

// Maximum and sum over the 64 lanes, returned in every lane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x = fmaxf(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  x = fmaxf(x, __builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false));  // row_ror 4
  x = fmaxf(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));  // row_ror 8
  x = fmaxf(x, xor16(x));
  return fmaxf(x, xor32(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false);
  x += xor16(x);
  return x + xor32(x);
}

__device__ __forceinline__ uint32_t pack_bf16(__bf16 lo, __bf16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// LDS of one wave, in floats: scores [C][64], partial sums [C][64],
// reference maxima [C] (padded to 32), the current column's probability
// pairs (hi parts [32], lo parts [32]), accumulators [C][64 lanes][D/32].
template <int D>
struct ValuSmem {
  static constexpr int C = kValuCols;
  static constexpr int NDT = D / 32;
  static constexpr int S_OFF = 0;
  static constexpr int L_OFF = C * 64;
  static constexpr int M_OFF = 2 * C * 64;
  static constexpr int P_OFF = M_OFF + 32;
  static constexpr int A_OFF = P_OFF + 64;
  static constexpr int WAVE = A_OFF + C * 64 * NDT;
  static_assert(A_OFF % 4 == 0 && P_OFF % 4 == 0, "16-byte LDS accesses");
  static_assert(4 * WAVE * 4 + C * D * 4 <= 160 * 1024, "LDS of one workgroup");
};

}  // namespace

template <int D, bool CAP>
__global__ __launch_bounds__(256, 1) void attn_valu_kernel(AttnArgs a) {
  using SM = ValuSmem<D>;
  constexpr int NK = D / 16;   // 16-byte loads of one sub-tile's K (and of its V)
  constexpr int NDT = D / 32;  // output dimensions per lane
  constexpr int NSUB_T = 128 / D > 1 ? 128 / D : 1;  // sub-tiles per planned tile
  __shared__ __align__(16) float smem[4 * SM::WAVE];
  // query parts: [column][D/2 pairs][hi pair, lo pair]
  __shared__ __align__(16) uint32_t qlds[kValuCols * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, r32 = lane & 31;
  const int w = blockIdx.x;
  const Chunk ch = chunk_of(a, w);
  const int h = ch.h, L = ch.L, n = ch.n;
  const int R = n * a.g;  // <= kValuCols (the planner's column cap)
  float* ws = smem + wave * SM::WAVE;
  float* sbuf = ws + SM::S_OFF;
  float* lbuf = ws + SM::L_OFF;
  float* mbuf = ws + SM::M_OFF;
  uint32_t* pbuf = reinterpret_cast<uint32_t*>(ws + SM::P_OFF);
  float* abuf = ws + SM::A_OFF;

  typedef __attribute__((address_space(4))) const int32_t cint32_t;
  cint32_t* trow = (cint32_t*)(a.table + (int64_t)ch.seq * a.max_bps);
  const int64_t head_off = (int64_t)h * 256 * D * 2;
  // sub-tiles [u0, u1) of the chunk (keys 32u .. 32u + 31); the wave takes
  // the pairs of consecutive sub-tiles wave, wave + 4, ...
  const int u0 = (ch.tlo + ch.t_begin) * NSUB_T, u1 = (ch.tlo + ch.t_end) * NSUB_T;
  const int npairs = (u1 - u0 + 1) / 2;
  const int cnt = wave < npairs ? (npairs - wave + 3) / 4 : 0;
  auto base = [&](int u) -> const uint8_t* {
    const int key0 = u * 32;
    return a.pool + (int64_t)trow[key0 >> 8] * a.lay.block_bytes + head_off + (int64_t)(key0 & 255) * D * 2;
  };
  // the k-th pair's sub-tiles; an odd chunk's last pair repeats its first
  // sub-tile, masked whole
  auto ua_of = [&](int k) { return u0 + 2 * (wave + 4 * k); };
  auto ub_of = [&](int k) { return min(ua_of(k) + 1, u1 - 1); };

  u32x4_t ka[NK], kb[NK], va[NK], vb[NK];
  auto load_k = [&](int k) {
    const uint8_t* pa = base(ua_of(k)) + a.lay.k_off;
    const uint8_t* pb = base(ub_of(k)) + a.lay.k_off;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      ka[j] = ld_stream(pa + j * 1024 + lane * 16);
      kb[j] = ld_stream(pb + j * 1024 + lane * 16);
    }
  };
  auto load_v = [&](int k) {
    const uint8_t* pa = base(ua_of(k)) + a.lay.v_off;
    const uint8_t* pb = base(ub_of(k)) + a.lay.v_off;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      va[j] = ld_stream(pa + j * 1024 + lane * 16);
      vb[j] = ld_stream(pb + j * 1024 + lane * 16);
    }
  };

  // the columns' queries as bf16 parts (hi = x rounded to bf16, lo = x - hi
  // rounded: x to about 2^-17): column c = row c / g, head c % g of this
  // slice; dword 2p (hi) and 2p + 1 (lo) of a column hold dimension pair p
  for (int i = threadIdx.x; i < R * (D / 2); i += 256) {
    const int c = i / (D / 2), p = i - c * (D / 2);
    const int ri = c / a.g, hj = c - ri * a.g;
    const float* qv = a.q + ((int64_t)(ch.qrow0 + ri) * a.hq + h * a.gq + a.head0 + hj) * D + 2 * p;
    const float x0 = qv[0], x1 = qv[1];
    const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1;
    qlds[c * D + 2 * p] = pack_bf16(h0, h1);
    qlds[c * D + 2 * p + 1] = pack_bf16((__bf16)(x0 - (float)h0), (__bf16)(x1 - (float)h1));
  }

  for (int c = 0; c < R; ++c) {
    if (lane == 0) mbuf[c] = NEG_INF;
    lbuf[c * 64 + lane] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) abuf[(c * 64 + lane) * NDT + dt] = 0.0f;
  }

  if (cnt > 0) load_k(0);
  __syncthreads();  // the query parts
  // Loads per iteration: this pair's values first (they arrive during the
  // key products), the next pair's keys after the key products (they arrive
  // during the value products), so the wait at the top of an iteration is
  // for the keys alone.
  for (int k = 0; k < cnt; ++k) {
    load_v(k);
    const int key0 = ua_of(k) * 32;
    const bool b_ok = ua_of(k) + 1 < u1;
    const int kp = key0 + lane;  // this lane's key (lanes 32..63: the second sub-tile)
    const bool kvalid = kp < L && (hh == 0 || b_ok);
    const bool full = b_ok && key0 + 64 <= L - n + 1 && (a.window == 0 || L - key0 <= a.window);

    // ---- scores, one key per lane
#pragma unroll
    for (int j = 0; j < NK; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto sw = __builtin_amdgcn_permlane32_swap(ka[j][e], kb[j][e], false, false);
        ka[j][e] = sw[0];  // dimension pair 8j + e
        kb[j][e] = sw[1];  // dimension pair 8j + 4 + e
      }
    {
      int hj = 0, ri = 0;
      for (int c = 0; c < R; ++c) {
        const u32x4_t* qv = reinterpret_cast<const u32x4_t*>(qlds + c * D);
        float x0 = 0.0f, x1 = 0.0f, x2 = 0.0f, x3 = 0.0f;
#pragma unroll
        for (int j = 0; j < NK; ++j) {
          // pairs 8j .. 8j + 7, both parts: dwords 16j .. 16j + 15, the same
          // address in every lane (LDS broadcast)
          const u32x4_t q0 = qv[4 * j], q1 = qv[4 * j + 1], q2 = qv[4 * j + 2], q3 = qv[4 * j + 3];
          const uint32_t qd[16] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3],
                                   q2[0], q2[1], q2[2], q2[3], q3[0], q3[1], q3[2], q3[3]};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x0 = dot2(ka[j][e], qd[2 * e], x0);
            x1 = dot2(ka[j][e], qd[2 * e + 1], x1);
            x2 = dot2(kb[j][e], qd[8 + 2 * e], x2);
            x3 = dot2(kb[j][e], qd[8 + 2 * e + 1], x3);
          }
        }
        float x = ((x0 + x2) + (x1 + x3)) * a.scale;
        if constexpr (CAP) x = a.softcap * tanh_nb(x * a.inv_softcap);
        x *= 1.4426950408889634f;  // log2 units: the softmax runs on exp2
        if (!full) {
          const int ppos = L - n + ri;
          const bool vis = kvalid && kp <= ppos && (a.window == 0 || ppos - kp < a.window);
          x = vis ? x : NEG_INF;
        }
        sbuf[c * 64 + lane] = x;
        const bool wrap = hj == a.g - 1;
        ri += wrap ? 1 : 0;
        hj = wrap ? 0 : hj + 1;
      }
    }
    // the K registers are free: the next pair's keys are requested now (the
    // last pair again after the end: an unconditional load keeps the
    // compiler's wait counts exact on every path)
    load_k(min(k + 1, cnt - 1));
    // keep the loads here (not sunk to the end of the iteration, where they
    // would be in flight for the next swap only)
    asm volatile("" ::: "memory");

    if (!full) {
      // value slots past the end (never written: any bits) and the repeated
      // sub-tile of an odd chunk contribute nothing.  V load v * NDT + dt,
      // dword t: keys 16v + 8(t >> 1) + 4hh + 2(t & 1) + {0, 1}.
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int j = 0; j < NK; ++j)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int v = j / NDT;
            const int kk = key0 + 32 * st + 16 * v + 8 * (t >> 1) + 4 * hh + 2 * (t & 1);
            const bool ok = st == 0 || b_ok;
            const uint32_t keep = (ok && kk < L ? 0x0000FFFFu : 0u) | (ok && kk + 1 < L ? 0xFFFF0000u : 0u);
            if (st == 0)
              va[j][t] &= keep;
            else
              vb[j][t] &= keep;
          }
    }

    // ---- per column: softmax, probability pairs, value products
    // This lane's key as a pair slot: sub-tile st, key m = 16v + 8(t >> 1) +
    // 4h + 2(t & 1) + b -> dword st * 16 + h * 8 + v * 4 + t, half b.
    const int pm = lane & 31;
    const int pslot = (lane >> 5) * 16 + ((pm >> 2) & 1) * 8 + (pm >> 4) * 4 + ((pm >> 3) & 1) * 2 + ((pm >> 1) & 1);
    for (int c = 0; c < R; ++c) {
      const float s = sbuf[c * 64 + lane];
      const float mt = wave_max(s);
      float m = mbuf[c];
      float alpha = 1.0f;
      if (mt > m + 8.0f) {  // the same decision in every lane
        alpha = fast_exp2(m - mt);  // 0 when nothing was seen yet
        m = mt;
      }
      const float m_use = m == NEG_INF ? 0.0f : m;
      const float p = fast_exp2(s - m_use);
      lbuf[c * 64 + lane] = fmaf(lbuf[c * 64 + lane], alpha, p);
      const __bf16 ph = (__bf16)p;
      const __bf16 pl = (__bf16)(p - (float)ph);
      // a key pair is two neighbouring lanes: the even lane stores both
      const int hb = __builtin_bit_cast(uint16_t, ph), lb = __builtin_bit_cast(uint16_t, pl);
      const int hn = __builtin_amdgcn_update_dpp(hb, hb, 0xB1, 0xF, 0xF, false);  // lane ^ 1
      const int ln = __builtin_amdgcn_update_dpp(lb, lb, 0xB1, 0xF, 0xF, false);
      if ((pm & 1) == 0) {
        pbuf[pslot] = (uint32_t)hb | ((uint32_t)hn << 16);
        pbuf[32 + pslot] = (uint32_t)lb | ((uint32_t)ln << 16);
      }
      // a wave's LDS accesses run in order: the reads below see these stores
      __builtin_amdgcn_wave_barrier();
      if (lane == 0) mbuf[c] = m;
      // this lane's key pairs: sub-tile st, dwords st * 16 + hh * 8 + 0..7
      u32x4_t phi[2][2], plo[2][2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          phi[st][v] = *reinterpret_cast<const u32x4_t*>(pbuf + st * 16 + hh * 8 + v * 4);
          plo[st][v] = *reinterpret_cast<const u32x4_t*>(pbuf + 32 + st * 16 + hh * 8 + v * 4);
        }
      float* ap = abuf + (c * 64 + lane) * NDT;
      float acc[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] = ap[dt] * alpha;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const u32x4_t vv = st == 0 ? va[v * NDT + dt] : vb[v * NDT + dt];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              acc[dt] = dot2(vv[t], phi[st][v][t], acc[dt]);
              acc[dt] = dot2(vv[t], plo[st][v][t], acc[dt]);
            }
          }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) ap[dt] = acc[dt];
      // the next column rewrites the probability pairs after these reads
      __builtin_amdgcn_wave_barrier();
    }
  }

  // ---- combine: sums over each wave (partial sums over its lanes,
  // accumulators over its halves), then the four waves through LDS
  for (int c = 0; c < R; ++c) {
    const float ls = wave_sum(lbuf[c * 64 + lane]);
    float x[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const float y = abuf[(c * 64 + lane) * NDT + dt];
      x[dt] = y + xor32(y);
    }
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) lbuf[c * 64] = ls;
    // column c's D sums, in the first D floats of its accumulator block
    if (hh == 0) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) abuf[c * 64 * NDT + 32 * dt + r32] = x[dt];
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  const bool whole = ch.k == 1 && !a.force_partial;
  float* slot = a.part + (int64_t)w * a.slot_stride;
  for (int idx = threadIdx.x; idx < R * D; idx += 256) {
    const int c = idx / D, dim = idx - c * D;
    float M = NEG_INF;
#pragma unroll
    for (int q = 0; q < 4; ++q) M = fmaxf(M, smem[q * SM::WAVE + SM::M_OFF + c]);
    const float mu = M == NEG_INF ? 0.0f : M;
    float ls = 0.0f, x = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* wq = smem + q * SM::WAVE;
      const float f = fast_exp2(wq[SM::M_OFF + c] - mu);
      ls += wq[SM::L_OFF + c * 64] * f;
      x += wq[SM::A_OFF + c * 64 * NDT + dim] * f;
    }
    const int ri = c / a.g, hj = c - ri * a.g;
    if (whole) {
      a.out[((int64_t)(ch.qrow0 + ri) * a.hq + h * a.gq + a.head0 + hj) * D + dim] = x / ls;
    } else {
      if (dim == 0) {
        slot[c] = M;
        slot[a.rpad + c] = ls;
      }
      slot[2 * a.rpad + (int64_t)c * D + dim] = x;
    }
  }
}

hipError_t launch_attn_valu(const AttnArgs& a, hipStream_t s) {
  if (a.n_wg <= 0) return hipSuccess;
  const int d = a.lay.d;
  if (a.lay.fmt != 1 || (d != 64 && d != 128) || a.rpad != 32) return hipErrorInvalidValue;
  const bool cap = a.softcap > 0.0f;
  dim3 grid(a.n_wg), block(256);
  if (d == 64) {
    if (cap)
      hipLaunchKernelGGL((attn_valu_kernel<64, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((attn_valu_kernel<64, false>), grid, block, 0, s, a);
  } else {
    if (cap)
      hipLaunchKernelGGL((attn_valu_kernel<128, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((attn_valu_kernel<128, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace svattn
