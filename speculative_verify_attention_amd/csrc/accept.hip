// accept.hip - acceptance of draft tokens after the verify forward, on gfx950.
//
// SwiftLM page, speculative-decoding passage: drafts are checked by
// rejection sampling as Leviathan et al. define it (the ratio P_target /
// P_draft decides each draft; a rejected position is re-sampled from the
// corrected distribution max(0, p - q)), so that the output follows the
// target distribution at non-zero temperature; greedy decoding takes the
// argmax and ignores the temperature.  Drafts without a distribution
// (n-gram drafts, AX Engine page, "Core Technical Architecture & Methods")
// are point masses.
//
// Three launches, all reading logits straight from HBM:
//  1. stats:  one workgroup per (row, 4096-logit chunk): chunk max, first
//             argmax and sum of exp((l - max) / T), coalesced 16-byte loads;
//  2. decide: one workgroup per (sequence, chunk) when sampling (one per
//             sequence when greedy).  Its waves combine the chunk statistics
//             of the sequence's rows in parallel, every thread then walks the
//             drafts from LDS and reaches the same decision; chunk 0 writes
//             the accepted count (greedy: and the token) and the draw's plan;
//             sampling: the workgroup sums the draw's weights over its chunk;
//  3. pick:   one workgroup per sampled sequence: a wave scan over the chunk
//             sums finds the chunk where u * total falls, a block scan over
//             runs of 8 logits finds the token.
// (Handing the draw to the last workgroup of step 2 instead of a third launch
// needs device-scope release/acquire between workgroups, which on this chip
// writes back and invalidates the L2 of every XCD; that costs more than a
// launch.)  One function computes every weight, so the draw sees the same
// values in the chunk sums and in the final scan.  Nothing is serial over the
// vocabulary: the only dependent chains are the drafts (at most 7) and the
// chunk count / 64.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.h"

namespace svattn {

namespace {

constexpr int kStatThreads = 256;  // stats: 16 logits per thread
constexpr int kThreads = 512;      // decide and pick: 8 logits per thread
constexpr int kWaves = kThreads / 64;
constexpr int kStatPer = kAcceptChunk / kStatThreads;
constexpr int kPer = kAcceptChunk / kThreads;
constexpr int kMaxRows = 2 * 7 + 1;  // target + draft rows of one sequence

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ float expt(float l, float m, float inv_t) { return __expf((l - m) * inv_t); }

// Wave-wide max with first index.
__device__ __forceinline__ void wave_argmax(float& v, int& idx) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(idx, o);
    if (better(ov, oi, v, idx)) {
      v = ov;
      idx = oi;
    }
  }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Block-wide sum in a fixed order (NT threads).
template <int NT>
__device__ __forceinline__ float block_sum(float x, float* sv) {
  x = wave_sum(x);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sv[wave] = x;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += sv[w];
  __syncthreads();
  return t;
}

// Logits of a chunk in the coalesced order: element e of thread t is token
// c0 + 4 (e/4 * NT + t) + e%4 with 16-byte loads (VEC: vocab % 4 == 0 and
// aligned rows), else c0 + e * NT + t.  Tokens past the vocabulary read -inf.
template <bool VEC, int NT>
__device__ __forceinline__ int chunk_token(int c0, int e) {
  if constexpr (VEC) return c0 + 4 * ((e >> 2) * NT + (int)threadIdx.x) + (e & 3);
  else return c0 + e * NT + (int)threadIdx.x;
}

__device__ __forceinline__ void put4(float* v, float4 f) {
  v[0] = f.x;
  v[1] = f.y;
  v[2] = f.z;
  v[3] = f.w;
}

template <bool VEC, int NT, int PER>
__device__ __forceinline__ void load_chunk(const float* src, int c0, int vocab, float (&v)[PER]) {
  if constexpr (VEC) {
#pragma unroll
    for (int g = 0; g < PER / 4; ++g) {
      const int x = c0 + 4 * (g * NT + (int)threadIdx.x);
      float4 f = float4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (x < vocab) f = *reinterpret_cast<const float4*>(src + x);  // vocab % 4 == 0: all four exist
      put4(v + 4 * g, f);
    }
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int x = c0 + e * NT + (int)threadIdx.x;
      v[e] = x < vocab ? src[x] : -INFINITY;
    }
  }
}

// The run of kPer consecutive tokens x0 .. x0 + kPer - 1 (x0 % kPer == 0).
template <bool VEC>
__device__ __forceinline__ void load_run(const float* src, int x0, int vocab, float (&v)[kPer]) {
  if constexpr (VEC) {
#pragma unroll
    for (int g = 0; g < kPer / 4; ++g) {
      const int x = x0 + 4 * g;
      float4 f = float4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (x < vocab) f = *reinterpret_cast<const float4*>(src + x);
      put4(v + 4 * g, f);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPer; ++e) v[e] = x0 + e < vocab ? src[x0 + e] : -INFINITY;
  }
}

// Weight of token x in the final draw (lt, lq: its target and draft logits).
__device__ __forceinline__ float draw_weight(const AcceptPlan& pl, float inv_t, float lt, float lq, int x) {
  const float p = expt(lt, pl.m_t, inv_t) * pl.is_t;
  if (pl.row_q >= 0) return fmaxf(0.0f, p - expt(lq, pl.m_q, inv_t) * pl.is_q);
  return x == pl.tok_q ? 0.0f : p;
}

// 1. Per (row, chunk) statistics.
template <bool VEC>
__global__ __launch_bounds__(kStatThreads) void accept_stats_kernel(AcceptArgs a) {
  __shared__ float sv[kStatThreads / 64];
  __shared__ int si[kStatThreads / 64];
  const int row = blockIdx.x / a.nch, chunk = blockIdx.x - row * a.nch;
  const float* src = row < a.rows_t ? a.target + (int64_t)row * a.vocab
                                    : a.draft + (int64_t)(row - a.rows_t) * a.vocab;
  const int c0 = chunk * kAcceptChunk;
  float v[kStatPer];
  load_chunk<VEC, kStatThreads, kStatPer>(src, c0, a.vocab, v);
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
#pragma unroll
  for (int e = 0; e < kStatPer; ++e) {
    const int x = chunk_token<VEC, kStatThreads>(c0, e);
    if (x < a.vocab && better(v[e], x, bv, bi)) {
      bv = v[e];
      bi = x;
    }
  }
  wave_argmax(bv, bi);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  bv = sv[0];
  bi = si[0];
#pragma unroll
  for (int w = 1; w < kStatThreads / 64; ++w)
    if (better(sv[w], si[w], bv, bi)) {
      bv = sv[w];
      bi = si[w];
    }
  __syncthreads();
  float sum = 0.0f;
  if (a.inv_t > 0.0f) {
    float t = 0.0f;
#pragma unroll
    for (int e = 0; e < kStatPer; ++e) t += expt(v[e], bv, a.inv_t);  // -inf -> 0
    sum = block_sum<kStatThreads>(t, sv);
  }
  if (threadIdx.x == 0) a.stats[blockIdx.x] = float4{bv, sum, __int_as_float(bi), 0.0f};
}

// Row statistics from its chunks (one wave): max, sum of exp((l - max)/T),
// first argmax.
struct RowStats {
  float m, s;
  int arg;
};

__device__ __forceinline__ RowStats row_stats(const AcceptArgs& a, int row) {
  const int lane = threadIdx.x & 63;
  const float4* st = a.stats + (int64_t)row * a.nch;
  const float4 none = float4{-INFINITY, 0.0f, __int_as_float(0x7FFFFFFF), 0.0f};
  // chunks lane and lane + 64 stay in registers (one round trip up to 128 chunks)
  const float4 x0 = lane < a.nch ? st[lane] : none;
  const float4 x1 = lane + 64 < a.nch ? st[lane + 64] : none;
  float m = x0.x;
  int arg = __float_as_int(x0.z);
  if (better(x1.x, __float_as_int(x1.z), m, arg)) {
    m = x1.x;
    arg = __float_as_int(x1.z);
  }
  for (int c = lane + 128; c < a.nch; c += 64) {
    const float4 x = st[c];
    if (better(x.x, __float_as_int(x.z), m, arg)) {
      m = x.x;
      arg = __float_as_int(x.z);
    }
  }
  wave_argmax(m, arg);
  float s = 0.0f;
  if (a.inv_t > 0.0f) {
    s = x0.y * expt(x0.x, m, a.inv_t) + x1.y * expt(x1.x, m, a.inv_t);  // -inf -> 0
    for (int c = lane + 128; c < a.nch; c += 64) {
      const float4 x = st[c];
      s += x.y * expt(x.x, m, a.inv_t);
    }
    s = wave_sum(s);
  }
  return RowStats{m, s, arg};
}

// The final draw of one sequence from its chunk sums fs: the smallest token x
// with cumulative weight > u * total (tokens in index order).  Every wave
// finds the chunk the same way from the same values; then a block scan over
// runs of kPer tokens.
template <bool VEC>
__device__ void draw_token(const AcceptArgs& a, const AcceptPlan& pl, int sidx, const float* fs) {
  __shared__ float wsum[kWaves];
  __shared__ int s_tok, s_first, s_last;  // crossing, first positive weight past it, last positive weight
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (threadIdx.x == 0) {
    s_tok = 0x7FFFFFFF;
    s_first = 0x7FFFFFFF;
    s_last = -1;
  }
  // inclusive scan of the chunk sums in chunk order, 64 at a time; total =
  // the last value, so u < 1 always lands inside
  auto scan64 = [&](float f) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float up = __shfl_up(f, o);
      if (lane >= o) f += up;
    }
    return f;
  };
  float rem = INFINITY;
  int pick = -1, lastpos = -1;
  if (a.nch <= 64) {  // one round trip
    const float f = lane < a.nch ? fs[lane] : 0.0f;
    const float inc = scan64(f);
    const float target = pl.u * __shfl(inc, 63);
    const uint64_t pos = __builtin_amdgcn_ballot_w64(f > 0.0f);
    if (pos) lastpos = 63 - __builtin_clzll(pos);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < a.nch && inc > target);
    if (hit) {
      pick = __builtin_ctzll(hit);
      rem = target - (__shfl(inc, pick) - __shfl(f, pick));
    }
  } else {
    float total = 0.0f;
    for (int base = 0; base < a.nch; base += 64)
      total += __shfl(scan64(base + lane < a.nch ? fs[base + lane] : 0.0f), 63);
    const float target = pl.u * total;
    float carry = 0.0f;
    for (int base = 0; base < a.nch; base += 64) {
      const int c = base + lane;
      const float f = c < a.nch ? fs[c] : 0.0f;
      const float inc = scan64(f);
      const uint64_t pos = __builtin_amdgcn_ballot_w64(f > 0.0f);
      if (pos) lastpos = base + 63 - __builtin_clzll(pos);
      if (pick < 0) {
        const uint64_t hit = __builtin_amdgcn_ballot_w64(c < a.nch && carry + inc > target);
        if (hit) {
          const int l = __builtin_ctzll(hit);
          pick = base + l;
          rem = target - (carry + __shfl(inc, l) - __shfl(f, l));
        }
      }
      carry += __shfl(inc, 63);
    }
  }
  if (pick < 0) pick = lastpos >= 0 ? lastpos : 0;  // rounding put u * total at or past the end

  // thread t owns tokens c0 + kPer t .. c0 + kPer t + kPer - 1
  const int c0 = pick * kAcceptChunk;
  const int x0 = c0 + kPer * (int)threadIdx.x;
  float lt[kPer], lq[kPer], w[kPer];
  load_run<VEC>(a.target + (int64_t)pl.row_t * a.vocab, x0, a.vocab, lt);
  if (pl.row_q >= 0) load_run<VEC>(a.draft + (int64_t)pl.row_q * a.vocab, x0, a.vocab, lq);
  float ts = 0.0f;
  int myfirst = -1, mylast = -1;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    w[e] = x0 + e < a.vocab ? draw_weight(pl, a.inv_t, lt[e], pl.row_q >= 0 ? lq[e] : 0.0f, x0 + e) : 0.0f;
    ts += w[e];
    if (w[e] > 0.0f) {
      if (myfirst < 0) myfirst = x0 + e;
      mylast = x0 + e;
    }
  }
  // exclusive block scan of the runs' sums in thread order
  float inc = ts;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float up = __shfl_up(inc, o);
    if (lane >= o) inc += up;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();  // also orders the s_tok / s_last initialisation before the atomics
  // Each run's start is exactly the previous run's end (the same fp32
  // values), so the runs tile [0, chunk sum) without gaps: the run whose
  // start is <= rem < end holds the crossing.  Its sequential sum may still
  // stop short of rem by rounding (the crossing within an ulp of a run
  // boundary); the crossing is then its last positive weight.
  float pre = 0.0f;  // sum of the earlier waves, in the order every wave adds it
  for (int w2 = 0; w2 < wave; ++w2) pre += wsum[w2];
  const float end = inc + pre;
  const float up = __shfl_up(end, 1);
  const float start = lane == 0 ? pre : up;
  // one atomic per wave: runs ascend with the lane, so the wave's last
  // positive weight is in its highest such lane, the first past the crossing
  // in its lowest
  const uint64_t has = __builtin_amdgcn_ballot_w64(mylast >= 0);
  if (has && lane == 63 - __builtin_clzll(has)) atomicMax(&s_last, mylast);
  const uint64_t past = __builtin_amdgcn_ballot_w64(start > rem && myfirst >= 0);
  if (past && lane == __builtin_ctzll(past)) atomicMin(&s_first, myfirst);
  if (start <= rem) {
    float cum = start;
    int t = -1;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      cum += w[e];
      if (t < 0 && cum > rem) t = x0 + e;
    }
    if (t < 0 && end > rem) t = mylast;
    if (t >= 0) atomicMin(&s_tok, t);
  }
  __syncthreads();
  if (threadIdx.x == 0)
    a.out_tok[sidx] = s_tok != 0x7FFFFFFF ? s_tok : s_first != 0x7FFFFFFF ? s_first : (s_last >= 0 ? s_last : c0);
}

// 2. Decide each sequence of the group; sum the draw's weights over a chunk.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void accept_decide_kernel(AcceptArgs a) {
  __shared__ float r_m[kMaxRows], r_is[kMaxRows], r_l[kMaxRows], r_u[kMaxRows];
  __shared__ int r_arg[kMaxRows], r_tok[kMaxRows];
  __shared__ float sv[kWaves];
  const bool samp = a.inv_t > 0.0f;
  const int per_seq = samp ? a.nch : 1;
  const int i = blockIdx.x / per_seq, chunk = blockIdx.x - i * per_seq;
  const int n = a.n[i], t0 = a.t0[i], d0 = a.d0[i];
  const int sidx = a.seq0 + i;
  const bool has_q = samp && a.draft != nullptr;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  // rows 0..n: target rows j; rows n+1 .. 2n: draft rows j (sampling with a
  // draft); one wave per row, all rows at once
  const int R = n + 1 + (has_q ? n : 0);
  for (int r = wave; r < R; r += kWaves) {
    const bool tr = r <= n;
    const int j = tr ? r : r - n - 1;
    const int grow = tr ? t0 + j : a.rows_t + d0 + j;
    const float* src = tr ? a.target + (int64_t)(t0 + j) * a.vocab : a.draft + (int64_t)(d0 + j) * a.vocab;
    const int tok = j < n ? a.drafts[d0 + j] : -1;
    const RowStats rs = row_stats(a, grow);
    const float l = (samp && tok >= 0 && tok < a.vocab) ? src[tok] : -INFINITY;
    if (lane == 0) {
      r_m[r] = rs.m;
      r_is[r] = samp ? 1.0f / rs.s : 0.0f;
      r_arg[r] = rs.arg;
      r_tok[r] = tok;
      r_l[r] = l;
      r_u[r] = (samp && tr) ? a.u[t0 + j] : 0.0f;
    }
  }
  __syncthreads();

  AcceptPlan pl{};
  pl.row_q = -1;
  pl.tok_q = -1;
  int acc = n, tok = -1;
  if (!samp) {
    for (int j = 0; j < n; ++j)
      if (r_tok[j] != r_arg[j]) {
        acc = j;
        tok = r_arg[j];
        break;
      }
    if (acc == n) tok = r_arg[n];
  } else {
    pl.mode = 1;
    pl.u = r_u[n];
    int rt = n, rq = -1;
    for (int j = 0; j < n; ++j) {
      const int d = r_tok[j];
      const bool valid = d >= 0 && d < a.vocab;
      const float pd = valid ? expt(r_l[j], r_m[j], a.inv_t) * r_is[j] : 0.0f;
      const float qd = (has_q && valid) ? expt(r_l[n + 1 + j], r_m[n + 1 + j], a.inv_t) * r_is[n + 1 + j] : 1.0f;
      if (!(r_u[j] * qd < pd)) {
        acc = j;
        rt = j;
        if (has_q) rq = n + 1 + j;
        else pl.tok_q = valid ? d : -1;
        break;
      }
    }
    pl.row_t = t0 + rt;
    pl.m_t = r_m[rt];
    pl.is_t = r_is[rt];
    if (rq >= 0) {
      pl.row_q = d0 + (rq - n - 1);
      pl.m_q = r_m[rq];
      pl.is_q = r_is[rq];
    }
  }
  if (chunk == 0 && threadIdx.x == 0) {
    a.out_acc[sidx] = acc;
    if (!samp) a.out_tok[sidx] = tok;
    else a.plan[sidx] = pl;
  }
  if (!samp) return;

  const int c0 = chunk * kAcceptChunk;
  float lt[kPer], lq[kPer];
  load_chunk<VEC, kThreads, kPer>(a.target + (int64_t)pl.row_t * a.vocab, c0, a.vocab, lt);
  if (pl.row_q >= 0) load_chunk<VEC, kThreads, kPer>(a.draft + (int64_t)pl.row_q * a.vocab, c0, a.vocab, lq);
  float t = 0.0f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int x = chunk_token<VEC, kThreads>(c0, e);
    if (x < a.vocab) t += draw_weight(pl, a.inv_t, lt[e], pl.row_q >= 0 ? lq[e] : 0.0f, x);
  }
  const float s = block_sum<kThreads>(t, sv);
  if (threadIdx.x == 0) a.fsum[(int64_t)sidx * a.nch + chunk] = s;
}

// 3. The draw of each sampled sequence.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void accept_pick_kernel(AcceptArgs a) {
  const int sidx = a.seq0 + (int)blockIdx.x;
  draw_token<VEC>(a, a.plan[sidx], sidx, a.fsum + (int64_t)sidx * a.nch);
}

bool vec_ok(const AcceptArgs& a) {
  return a.vocab % 4 == 0 && reinterpret_cast<uintptr_t>(a.target) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(a.draft) % 16 == 0;
}

}  // namespace

hipError_t launch_accept_stats(const AcceptArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)(a.rows_t + a.rows_d) * a.nch;
  if (blocks <= 0) return hipSuccess;
  if (vec_ok(a))
    hipLaunchKernelGGL(accept_stats_kernel<true>, dim3((unsigned)blocks), dim3(kStatThreads), 0, s, a);
  else
    hipLaunchKernelGGL(accept_stats_kernel<false>, dim3((unsigned)blocks), dim3(kStatThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_accept_group(const AcceptArgs& a, hipStream_t s) {
  if (a.count <= 0) return hipSuccess;
  const bool samp = a.inv_t > 0.0f, vec = vec_ok(a);
  const dim3 grid(samp ? a.count * a.nch : a.count);
  if (vec) hipLaunchKernelGGL(accept_decide_kernel<true>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(accept_decide_kernel<false>, grid, dim3(kThreads), 0, s, a);
  if (samp) {
    if (vec) hipLaunchKernelGGL(accept_pick_kernel<true>, dim3(a.count), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL(accept_pick_kernel<false>, dim3(a.count), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace svattn
