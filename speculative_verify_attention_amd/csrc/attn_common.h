// attn_common.h - device helpers shared by the verify-attention kernels:
// vector types, exp2, the branch-free tanh of the soft cap, work lookup
// (which chunk of which (sequence, kv head) pair a workgroup owns), the
// online-softmax state and update, and the combine/store epilogue.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace svattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define NEG_INF (-__builtin_inff())

// Depth of the register ring of 16 KiB tiles (tiles in flight + 1), and the
// waves per SIMD the bf16 kernels at d <= 128 are compiled for.
#ifndef SVATTN_NBUF
#define SVATTN_NBUF 2
#endif
#ifndef SVATTN_BF16_WAVES
#define SVATTN_BF16_WAVES 1
#endif

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Loads of the cache stream: every stored byte is read once per call, so
// the loads carry the non-temporal hint (global_load ... nt).  Measured on
// MI355X over a 2 GiB buffer, the same grid-stride pass reads 7.2 TB/s with
// the hint against 6.5 TB/s without.
__device__ __forceinline__ u32x4_t ld_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ uint32_t ld_stream_u32(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// tanh without branches, for the soft cap: the odd Taylor polynomial to x^9
// below |x| = 0.25 (truncation below 1e-8 relative there) and
// 1 - 2 / (e^{2|x|} + 1) above, with the hardware reciprocal (1 ulp); the
// subtraction loses a few ulp of 1, about 1e-7 absolute, near the switch.
__device__ __forceinline__ float tanh_nb(float x) {
  const float ax = fabsf(x);
  const float x2 = x * x;
  float p = 62.0f / 2835.0f;
  p = fmaf(p, x2, -17.0f / 315.0f);
  p = fmaf(p, x2, 2.0f / 15.0f);
  p = fmaf(p, x2, -1.0f / 3.0f);
  const float small = fmaf(x * x2, p, x);
  const float e = fast_exp2(ax * 2.8853900817779268f);  // e^{2|x|}
  const float big = copysignf(fmaf(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f), x);
  return ax < 0.25f ? small : big;
}

// Value of lane l ^ 32: one lane-swap between the wave's halves (no LDS
// round trip).
__device__ __forceinline__ float xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// Online-softmax state of one lane: column c's running reference max m (log2
// units, equal in both half-waves), this lane's partial sum l, and its part
// of the column's O^T accumulator.
template <int D>
struct ColState {
  float m, l;
  f32x16_t acc[D / 32];
};

// Online-softmax update of one tile's scores p (log2 units, -inf = masked):
// row maxima over the two half-waves, lazy move of the reference max (only
// when the tile max exceeds it by more than tau, 8 by default, so
// probabilities stay below 2^tau and rescales are rare), then
// p <- 2^(p - m) and the running sum.
template <int D, int NSUB>
__device__ __forceinline__ void softmax_update(ColState<D>& cs, float (&p)[NSUB][16], float tau = 8.0f,
                                               float mul = 1.0f) {
  // p holds scores in log2 units times 1 / mul (mul > 0): the multiply is
  // folded into the max and into the exponent's argument
  float mt = NEG_INF;
#pragma unroll
  for (int st = 0; st < NSUB; ++st)
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, p[st][r]);
  mt = fmaxf(mt, xor32(mt)) * mul;
  const bool up = mt > cs.m + tau;
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(up) != 0, 0)) {
    // lanes that move: alpha = 2^(m_old - m_new), 0 when nothing was seen yet;
    // lanes that stay keep alpha = 1 (their m may still be -inf)
    const float alpha = up ? fast_exp2(cs.m - mt) : 1.0f;
    cs.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      // d = 256: the accumulators live in accumulation registers.  Taking
      // them from there and handing the scaled values back inside this
      // rarely taken branch (the empty asm statements pin both ends to it)
      // keeps the compiler from holding a vector-register copy of every
      // accumulator across the whole loop for the multiply.
      f32x16_t t = cs.acc[dt];
      if constexpr (D > 128) asm volatile("" : "+a"(t));
      t *= alpha;
      if constexpr (D > 128) asm volatile("" : "+a"(t));
      cs.acc[dt] = t;
    }
    cs.m = up ? mt : cs.m;
  }
  const float m_use = cs.m == NEG_INF ? 0.0f : cs.m;
  float lsum = 0.0f;
#pragma unroll
  for (int st = 0; st < NSUB; ++st)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(fmaf(p[st][r], mul, -m_use));
      p[st][r] = e;
      lsum += e;
    }
  cs.l += lsum;
}

// Chunk of workgroup w: sequence index s (cache sequence seq, n query rows
// from query row qrow0, L positions), kv head h, chunk `part` of k, tiles
// [t_begin, t_end) of the pair's nt (empty when pending device rollbacks
// left fewer tiles than the host planned for).
struct Chunk {
  int s, seq, qrow0, n, h, k, part, L, nt, tlo, t_begin, t_end;
};

// The per-sequence fields sit in the kernel arguments, which the first
// reads fetch from memory.  Every lane reads the fields of sequences lane
// and lane + 64 at once (coalesced, one round trip); the workgroup's
// sequence is the number of sequences whose first workgroup is <= w, less
// one (wg_base ascends), and its fields are then taken from the lane that
// read them.  A search over wg_base with scalar reads would wait for one
// round trip per step, then one more for the fields.
__device__ __forceinline__ Chunk chunk_of(const AttnArgs& a, int w) {
  constexpr int NF = 6;  // wg_base, ksplit, len, nrows, seq, qrow0
  static_assert(kMaxAttnSeqs >= 64, "one sequence per lane");
  const int lane = threadIdx.x & 63;
  const int ns = a.n_seqs;
  int f0[NF], f1[NF];
  // unconditional reads inside the arrays (entries past n_seqs are ignored),
  // so that the compiler issues them together
  auto fetch = [&](int i, int (&f)[NF]) {
    f[0] = a.wg_base[i];
    f[1] = a.ksplit[i];
    f[2] = a.len[i];
    f[3] = a.nrows[i];
    f[4] = a.seq[i];
    f[5] = a.qrow0[i];
  };
  fetch(lane, f0);
  const bool two = ns > 64;
  if (two) fetch(min(lane + 64, kMaxAttnSeqs - 1), f1);
  const uint64_t b0 = __ballot(lane < ns && f0[0] <= w);
  const uint64_t b1 = two ? __ballot(lane + 64 < ns && f1[0] <= w) : 0ull;
  const int s = __popcll(b0) + __popcll(b1) - 1;
  int v[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j)
    v[j] = s < 64 ? __builtin_amdgcn_readlane(f0[j], s) : __builtin_amdgcn_readlane(f1[j], s - 64);
  Chunk c;
  c.s = s;
  c.k = v[1];
  c.seq = v[4];
  c.qrow0 = v[5];
  c.n = v[3];
  const int local = w - v[0];
  c.h = local / c.k;
  const int part = local - c.h * c.k;
  c.part = part;
  const int L = a.roll ? v[2] - a.roll[c.seq] : v[2], n = c.n;
  c.L = L;
  const int tk = a.tile_keys;
  const int klo = a.window > 0 ? max(0, L - n - a.window + 1) : 0;
  c.tlo = klo / tk;
  c.nt = (L + tk - 1) / tk - c.tlo;
  const int cs = (c.nt + c.k - 1) / c.k;
  c.t_begin = part * cs;
  c.t_end = min(c.nt, c.t_begin + cs);
  return c;
}

// Combine the token lanes of each column group through LDS, then either
// write the normalized output (the pair was one chunk) or the chunk's
// partial (m, l, acc) into its slot for the merge.
// NW waves per workgroup: NCT column groups of NW / NCT token-lane waves.
// Token lanes that are not a power of two first fold the lanes past the
// largest power of two P into the first TL - P, then halve P down to 1.
template <int D, int NCT, int NW = 4>
struct CombineBuf {
  static constexpr int TL = NW / NCT;
  static constexpr int P = TL >= 8 ? 8 : TL >= 4 ? 4 : TL >= 2 ? 2 : 1;  // TL <= 15
  static constexpr int SLOTS = (TL - P > P / 2 ? TL - P : P / 2) > 0 ? (TL - P > P / 2 ? TL - P : P / 2) : 1;
  static constexpr int CSTRIDE = D * 32 + 64;  // floats per combine slot
  static constexpr int FLOATS = NCT * SLOTS * CSTRIDE;
  static_assert(TL >= 1 && TL < 16, "token lanes");
};

// DS, dim0: the output's head size and the first dimension this state
// holds (a state may hold a part of the dimensions); write_ml: this call
// stores the partial slot's maxima and sums (one of the parts does).
template <int D, int NCT, int NW = 4, int DS = D>
__device__ __forceinline__ void combine_and_store(ColState<D>& cs, float* cbuf, const AttnArgs& a, int w, int k,
                                                  int s, int h, int row_i, int head_j, bool col_ok, int lane,
                                                  int ct, int tl, int dim0 = 0, bool write_ml = true) {
  constexpr int TL = NW / NCT;
  constexpr int P = CombineBuf<D, NCT, NW>::P;
  constexpr int SLOTS = CombineBuf<D, NCT, NW>::SLOTS;
  constexpr int NDT = D / 32;
  constexpr int CSTRIDE = CombineBuf<D, NCT, NW>::CSTRIDE;
  const int col = lane & 31, hh = lane >> 5;
  const int c = ct * 32 + col;
  cs.l += xor32(cs.l);
  auto put = [&](int idx) {
    float* slot = cbuf + (ct * SLOTS + idx) * CSTRIDE;
    if (hh == 0) {
      slot[col] = cs.m;
      slot[32 + col] = cs.l;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) slot[64 + (dt * 16 + r) * 64 + lane] = cs.acc[dt][r];
  };
  auto fold = [&](int idx) {
    const float* slot = cbuf + (ct * SLOTS + idx) * CSTRIDE;
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
  };
  if constexpr (TL > P) {
    if (tl >= P) put(tl - P);
    __syncthreads();
    if (tl < TL - P) fold(tl);
    __syncthreads();
  }
#pragma unroll
  for (int half = P / 2; half >= 1; half >>= 1) {
    if (tl >= half && tl < 2 * half) put(tl - half);
    __syncthreads();
    if (tl < half) fold(tl);
    if (half > 1) __syncthreads();
  }

  if (tl == 0 && col_ok) {
    if (k == 1 && !a.force_partial) {
      const float inv = 1.0f / cs.l;
      float* o = a.out + ((int64_t)(a.qrow0[s] + row_i) * a.hq + h * a.gq + a.head0 + head_j) * DS + dim0;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4_t v = {cs.acc[dt][4 * j] * inv, cs.acc[dt][4 * j + 1] * inv, cs.acc[dt][4 * j + 2] * inv,
                       cs.acc[dt][4 * j + 3] * inv};
          *reinterpret_cast<f32x4_t*>(o + 32 * dt + 8 * j + 4 * hh) = v;
        }
    } else {
      float* slot = a.part + (int64_t)w * a.slot_stride;
      if (hh == 0 && write_ml) {
        slot[c] = cs.m;
        slot[a.rpad + c] = cs.l;
      }
      float* acc = slot + 2 * a.rpad + (int64_t)c * DS + dim0;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4_t v = {cs.acc[dt][4 * j], cs.acc[dt][4 * j + 1], cs.acc[dt][4 * j + 2], cs.acc[dt][4 * j + 3]};
          *reinterpret_cast<f32x4_t*>(acc + 32 * dt + 8 * j + 4 * hh) = v;
        }
    }
  }
}

}  // namespace svattn
