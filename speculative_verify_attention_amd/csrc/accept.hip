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
// Four launches, all reading logits straight from HBM with coalesced loads:
//  1. stats:  one workgroup per (row, 4096-logit chunk): chunk max, first
//             argmax and sum of exp((l - max) / T);
//  2. decide: one wave per sequence: combine the chunk statistics of the
//             rows it needs, walk the drafts, write the accepted count (and
//             the token, for greedy) and the plan of the final draw;
//  3. sums:   one workgroup per (sequence, chunk): chunk sums of the final
//             draw's weights;
//  4. pick:   one workgroup per sequence: the chunk where u * total falls,
//             then the token inside it.
// Every weight is computed by one function in kernels 3 and 4, so the draw
// sees the same values in both.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.h"

namespace svattn {

namespace {

constexpr int kThreads = 256;
constexpr int kPer = kAcceptChunk / kThreads;  // logits per thread per chunk

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Block-wide max with first index, then (if wanted) sum; 256 threads.
__device__ __forceinline__ void block_argmax(float& v, int& idx, float* sv, int* si) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(idx, o);
    if (better(ov, oi, v, idx)) {
      v = ov;
      idx = oi;
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sv[wave] = v;
    si[wave] = idx;
  }
  __syncthreads();
  v = sv[0];
  idx = si[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w)
    if (better(sv[w], si[w], v, idx)) {
      v = sv[w];
      idx = si[w];
    }
  __syncthreads();
}

__device__ __forceinline__ float block_sum(float x, float* sv) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sv[wave] = x;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) t += sv[w];  // fixed order
  __syncthreads();
  return t;
}

__device__ __forceinline__ float expt(float l, float m, float inv_t) { return __expf((l - m) * inv_t); }

// Weight of token x in the final draw of plan pl.
__device__ __forceinline__ float draw_weight(const AcceptArgs& a, const AcceptPlan& pl, int x) {
  const float p = expt(a.target[(int64_t)pl.row_t * a.vocab + x], pl.m_t, a.inv_t) / pl.s_t;
  if (pl.row_q >= 0) {
    const float q = expt(a.draft[(int64_t)pl.row_q * a.vocab + x], pl.m_q, a.inv_t) / pl.s_q;
    return fmaxf(0.0f, p - q);
  }
  return x == pl.tok_q ? 0.0f : p;
}

// 1. Per (row, chunk) statistics.
__global__ __launch_bounds__(kThreads) void accept_stats_kernel(AcceptArgs a) {
  __shared__ float sv[kThreads / 64];
  __shared__ int si[kThreads / 64];
  const int row = blockIdx.x / a.nch, chunk = blockIdx.x - row * a.nch;
  const float* src = row < a.rows_t ? a.target + (int64_t)row * a.vocab
                                    : a.draft + (int64_t)(row - a.rows_t) * a.vocab;
  const int c0 = chunk * kAcceptChunk;
  float v[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int x = c0 + e * kThreads + threadIdx.x;  // each load: 256 consecutive logits
    v[e] = x < a.vocab ? src[x] : -INFINITY;
  }
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int x = c0 + e * kThreads + threadIdx.x;
    if (x < a.vocab && better(v[e], x, bv, bi)) {
      bv = v[e];
      bi = x;
    }
  }
  block_argmax(bv, bi, sv, si);
  float sum = 0.0f;
  if (a.inv_t > 0.0f) {
    float t = 0.0f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) t += expt(v[e], bv, a.inv_t);  // -inf -> 0
    sum = block_sum(t, sv);
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
  float m = -INFINITY;
  int arg = 0x7FFFFFFF;
  for (int c = lane; c < a.nch; c += 64) {
    const float4 x = st[c];
    if (better(x.x, __float_as_int(x.z), m, arg)) {
      m = x.x;
      arg = __float_as_int(x.z);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float om = __shfl_xor(m, o);
    const int oa = __shfl_xor(arg, o);
    if (better(om, oa, m, arg)) {
      m = om;
      arg = oa;
    }
  }
  float s = 0.0f;
  if (a.inv_t > 0.0f) {
    for (int c = lane; c < a.nch; c += 64) {
      const float4 x = st[c];
      s += x.y * expt(x.x, m, a.inv_t);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  }
  return RowStats{m, s, arg};
}

// 2. Decide each sequence of the group.
__global__ __launch_bounds__(64) void accept_decide_kernel(AcceptArgs a) {
  const int i = blockIdx.x;  // sequence within the group
  const int n = a.n[i], t0 = a.t0[i], d0 = a.d0[i];
  const int sidx = a.seq0 + i;
  AcceptPlan pl{};
  pl.mode = 0;
  pl.row_q = -1;
  pl.tok_q = -1;
  int acc = n, tok = -1;
  if (a.inv_t == 0.0f) {
    for (int j = 0; j < n; ++j) {
      const int am = row_stats(a, t0 + j).arg;
      if (a.drafts[d0 + j] != am) {
        acc = j;
        tok = am;
        break;
      }
    }
    if (acc == n) tok = row_stats(a, t0 + n).arg;
  } else {
    pl.mode = 1;
    pl.u = a.u[t0 + n];
    bool rejected = false;
    for (int j = 0; j < n && !rejected; ++j) {
      const RowStats rt = row_stats(a, t0 + j);
      const int d = a.drafts[d0 + j];
      const bool valid = d >= 0 && d < a.vocab;
      const float pd = valid ? expt(a.target[(int64_t)(t0 + j) * a.vocab + d], rt.m, a.inv_t) / rt.s : 0.0f;
      float qd = 1.0f;
      RowStats rq{0.0f, 1.0f, 0};
      if (a.draft) {
        rq = row_stats(a, a.rows_t + d0 + j);
        if (valid) qd = expt(a.draft[(int64_t)(d0 + j) * a.vocab + d], rq.m, a.inv_t) / rq.s;
      }
      if (!(a.u[t0 + j] * qd < pd)) {
        rejected = true;
        acc = j;
        pl.row_t = t0 + j;
        pl.m_t = rt.m;
        pl.s_t = rt.s;
        if (a.draft) {
          pl.row_q = d0 + j;
          pl.m_q = rq.m;
          pl.s_q = rq.s;
        } else {
          pl.tok_q = valid ? d : -1;
        }
      }
    }
    if (!rejected) {
      const RowStats rt = row_stats(a, t0 + n);
      pl.row_t = t0 + n;
      pl.m_t = rt.m;
      pl.s_t = rt.s;
    }
  }
  if (threadIdx.x == 0) {
    a.out_acc[sidx] = acc;
    if (pl.mode == 0) a.out_tok[sidx] = tok;
    a.plan[sidx] = pl;
  }
}

// 3. Chunk sums of the final draw's weights.
__global__ __launch_bounds__(kThreads) void accept_sums_kernel(AcceptArgs a) {
  __shared__ float sv[kThreads / 64];
  const int i = blockIdx.x / a.nch, chunk = blockIdx.x - i * a.nch;
  const int sidx = a.seq0 + i;
  const AcceptPlan pl = a.plan[sidx];
  if (pl.mode == 0) return;
  const int c0 = chunk * kAcceptChunk;
  float t = 0.0f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int x = c0 + e * kThreads + threadIdx.x;
    if (x < a.vocab) t += draw_weight(a, pl, x);
  }
  const float s = block_sum(t, sv);
  if (threadIdx.x == 0) a.fsum[(int64_t)sidx * a.nch + chunk] = s;
}

// 4. The token: smallest x with cumulative weight > u * total (tokens in
// index order); chunk by chunk, then inside the chunk.
__global__ __launch_bounds__(kThreads) void accept_pick_kernel(AcceptArgs a) {
  __shared__ int s_chunk;
  __shared__ float s_rem;
  __shared__ float part[kThreads];
  __shared__ int s_tok, s_last;
  const int i = blockIdx.x;
  const int sidx = a.seq0 + i;
  const AcceptPlan pl = a.plan[sidx];
  if (pl.mode == 0) return;
  const float* fs = a.fsum + (int64_t)sidx * a.nch;
  if (threadIdx.x == 0) {
    float total = 0.0f;
    for (int c = 0; c < a.nch; ++c) total += fs[c];
    const float target = pl.u * total;
    float cum = 0.0f;
    int pick = -1, lastpos = 0;
    float rem = 0.0f;
    for (int c = 0; c < a.nch; ++c) {
      if (fs[c] > 0.0f) lastpos = c;
      if (pick < 0 && cum + fs[c] > target) {
        pick = c;
        rem = target - cum;
      }
      cum += fs[c];
    }
    if (pick < 0) {  // rounding put u * total at or past the end
      pick = lastpos;
      rem = INFINITY;
    }
    s_chunk = pick;
    s_rem = rem;
    s_tok = 0x7FFFFFFF;
    s_last = -1;
  }
  __syncthreads();
  const int c0 = s_chunk * kAcceptChunk;
  const float rem = s_rem;
  // thread t owns logits c0 + kPer t .. +kPer (contiguous: a sequential scan)
  float w[kPer];
  float t = 0.0f;
  int lastpos = -1;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int x = c0 + kPer * threadIdx.x + e;
    w[e] = x < a.vocab ? draw_weight(a, pl, x) : 0.0f;
    t += w[e];
    if (w[e] > 0.0f) lastpos = x;
  }
  part[threadIdx.x] = t;
  if (lastpos >= 0) atomicMax(&s_last, lastpos);
  __syncthreads();
  if (threadIdx.x == 0) {  // exclusive scan in thread order
    float cum = 0.0f;
    for (int k = 0; k < kThreads; ++k) {
      const float x = part[k];
      part[k] = cum;
      cum += x;
    }
  }
  __syncthreads();
  float cum = part[threadIdx.x];
  if (cum <= rem) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      cum += w[e];
      if (cum > rem) {
        atomicMin(&s_tok, c0 + kPer * threadIdx.x + e);
        break;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.out_tok[sidx] = s_tok != 0x7FFFFFFF ? s_tok : (s_last >= 0 ? s_last : c0);
}

}  // namespace

hipError_t launch_accept_stats(const AcceptArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)(a.rows_t + a.rows_d) * a.nch;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(accept_stats_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_accept_group(const AcceptArgs& a, hipStream_t s) {
  if (a.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(accept_decide_kernel, dim3(a.count), dim3(64), 0, s, a);
  if (a.inv_t > 0.0f) {
    hipLaunchKernelGGL(accept_sums_kernel, dim3(a.count * a.nch), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(accept_pick_kernel, dim3(a.count), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace svattn
