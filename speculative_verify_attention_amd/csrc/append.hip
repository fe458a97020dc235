// append.hip - the write side of the cache on gfx950:
//  * block-table update (new blocks of an append become visible to readers);
//  * slice-update of new K/V positions into their blocks (fp32 / bf16);
//  * quantize-on-append for the compressed format, and the same encoder as a
//    stand-alone pass (kv_encode).
//
// AX Engine page, "Core Technical Architecture & Methods": the cache grows by
// slice-updates into preallocated buffers.  SwiftLM page, TurboQuant KV-cache
// compression passage: keys get 3-bit Lloyd-Max codes plus a 1-bit QJL
// residual, values 3-bit codes only, encoded natively.
//
// The encoder works in double precision, one wavefront per vector; the
// rotation is a fast Walsh-Hadamard transform done in registers with
// cross-lane exchanges.  It is off the throughput path (a few vectors per
// sequence per step), so it is written for exactness, not speed.
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "lanes.h"
#include "qprep.h"

namespace svattn {

PoolLayout make_layout(int fmt, int hkv, int d) {
  PoolLayout L{};
  L.fmt = fmt;
  L.hkv = hkv;
  L.d = d;
  if (fmt == 2) {
    L.block_bytes = (int64_t)hkv * 8 * tq3_sub_bytes(d);
  } else {
    int64_t e = fmt == 0 ? 4 : 2;
    L.k_off = 0;
    L.v_off = (int64_t)hkv * 256 * d * e;
    L.block_bytes = 2 * L.v_off;
  }
  return L;
}

// ---- block-table update -------------------------------------------------------

__global__ void table_update_kernel(TableUpdateArgs a) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < a.count) a.table[a.index[i]] = a.block[i];
}

hipError_t launch_table_update(const TableUpdateArgs& a, hipStream_t s) {
  if (a.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(table_update_kernel, dim3((a.count + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---- device-side rollback --------------------------------------------------------

// One thread per entry; sequence ids are distinct within a call, so no two
// threads touch one counter.
__global__ void rollback_kernel(RollbackArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.count) return;
  const int n = a.n_draft[i];
  const int r = n - min(max(a.accepted[i], 0), n);
  a.roll[a.seq[i]] += r;
}

hipError_t launch_rollback(const RollbackArgs& a, hipStream_t s) {
  if (a.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(rollback_kernel, dim3((a.count + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

// A fill kernel rather than hipMemsetAsync, so that callers may capture it.
__global__ void fill_zero_kernel(int32_t* p, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_fill_zero(int32_t* p, int32_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

// ---- helpers --------------------------------------------------------------------

// First position of segment seg after any pending device rollback.
__device__ inline int seg_pos0(const AppendArgs& a, int seg) {
  return a.roll ? a.pos0[seg] - a.roll[a.seq[seg]] : a.pos0[seg];
}

__device__ inline int find_seg(const int32_t* unit0, int n_segs, int unit) {
  int lo = 0, hi = n_segs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (unit0[mid] <= unit)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}


// IEEE half (bits) of a non-negative double, nearest-even, saturating at 65504.
__device__ inline uint16_t half_rne(double x, uint32_t* sat) {
  if (!(x == x)) return 0x7E00;
  if (x >= 65520.0) {
    *sat = 1;
    return 0x7BFF;
  }
  if (x < 0x1p-14) return (uint16_t)__builtin_rint(x * 0x1p24);
  int e = ilogb(x);
  double m = __builtin_rint(ldexp(x, 10 - e));
  if (m == 2048.0) {
    m = 1024.0;
    e += 1;
  }
  if (e + 15 >= 31) {
    *sat = 1;
    return 0x7BFF;
  }
  return (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

__device__ inline double half_value(uint16_t h) {
  int e = (h >> 10) & 31, f = h & 1023;
  return e == 0 ? (double)f * 0x1p-24 : ldexp((double)(f + 1024), e - 25);
}

// Encoded form of one vector, spread over a wavefront: lane l owns
// dimensions l*E .. l*E+E-1 (E = D / 64).
template <int D>
struct EncOut {
  static constexpr int E = D / 64;
  uint8_t code[E];
  uint8_t bit[E];
  uint16_t n16, g16;
};

// A lane's E = D / 64 values of a source vector (dimensions lane*E ..).
template <int D>
struct SrcVec {
  float x[D / 64];
  __device__ __forceinline__ void load(const float* __restrict__ src) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) x[e] = src[lane * (D / 64) + e];
  }
};

// Encode one vector (its values already loaded by every lane) with one full
// wavefront.  rbuf: this wave's D doubles of LDS.
template <int D>
__device__ __forceinline__ void encode_vector(const SrcVec<D>& xs, bool is_key, const int8_t* __restrict__ signs,
                              const float* __restrict__ s_t, const double* thr, const double* lev16,
                              double* rbuf, EncOut<D>& o, uint32_t* sat) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  double v[E];
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    double xi = (double)xs.x[e];
    ss += xi * xi;
    v[e] = signs[lane * E + e] < 0 ? -xi : xi;  // D x
  }
  ss = lanes_sum(ss);
  const double n = sqrt(ss);
  // zx = H (D x): Walsh-Hadamard butterflies; in-lane stages first, then
  // cross-lane stages (partner lane = lane ^ (h / E)).
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (!(e & h)) {
        double a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
    }
  }
  wht_lanes(v, lane);
  // z = sqrt(d) * Pi x / n = zx / n; code = #thresholds <= z.
  uint32_t s = 0;
  const uint16_t n16 = half_rne(n, &s);
  const double n16v = half_value(n16);
  const double inv_sqrt_d = 1.0 / sqrt((double)D);
  double r[E];
  double rr = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    double z = n > 0.0 ? v[e] / n : 0.0;
    int c = 0;
#pragma unroll
    for (int j = 0; j < 7; ++j) c += (thr[j] <= z) ? 1 : 0;
    o.code[e] = (uint8_t)c;
    // residual in the rotated frame: Pi x - n16 * c16[code] / sqrt(d)
    r[e] = (v[e] - n16v * lev16[c]) * inv_sqrt_d;
    rr += r[e] * r[e];
  }
  o.n16 = n16;
  o.g16 = 0;
  if (is_key) {
    rr = lanes_sum(rr);
    o.g16 = half_rne(sqrt(rr), &s);
    // proj = S r: every lane needs all of r, so pass it through LDS.
#pragma unroll
    for (int e = 0; e < E; ++e) rbuf[lane * E + e] = r[e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // four partial sums per output (rows j = u mod 4), so that four chains
    // of dependent fp64 fmas run side by side instead of one of length D;
    // unrolled so that many rows of S^T are in flight at once
    double proj[4][E];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) proj[u][e] = 0.0;
#pragma unroll 4
    for (int j = 0; j < D; j += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double rj = rbuf[j + u];
#pragma unroll
        for (int e = 0; e < E; ++e) proj[u][e] = fma((double)s_t[(j + u) * D + lane * E + e], rj, proj[u][e]);
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) o.bit[e] = ((proj[0][e] + proj[1][e]) + (proj[2][e] + proj[3][e])) >= 0.0 ? 1 : 0;
    // keep rbuf stable until every lane has read it before a later reuse
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) o.bit[e] = 0;
  }
  if (s) *sat = 1;
}

// Write the key nibbles of one encoded vector: byte b of the record holds
// dims 2b (low nibble) and 2b+1 (high nibble).
template <int D>
__device__ inline void store_key_nibbles(uint8_t* dst, const EncOut<D>& o) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  if constexpr (E == 1) {
    uint32_t nib = (uint32_t)(o.code[0] | (o.bit[0] << 3));
    uint32_t hi = __shfl_down(nib, 1);
    if ((lane & 1) == 0) dst[lane >> 1] = (uint8_t)(nib | (hi << 4));
  } else {
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      uint32_t lo = o.code[e] | (o.bit[e] << 3);
      uint32_t hi = o.code[e + 1] | (o.bit[e + 1] << 3);
      dst[(lane * E + e) >> 1] = (uint8_t)(lo | (hi << 4));
    }
  }
}

__device__ inline void store_half(uint8_t* p, uint16_t h) {
  p[0] = (uint8_t)(h & 0xFF);
  p[1] = (uint8_t)(h >> 8);
}

// ---- plain slice-update ----------------------------------------------------------

template <typename T, int FMT>
__global__ __launch_bounds__(64) void append_plain_kernel(AppendArgs a) {
  const int unit = blockIdx.x;  // one source row
  const int h = blockIdx.y;
  const int seg = find_seg(a.unit0, a.n_segs, unit);
  const int r = unit - a.unit0[seg];
  const int pos = seg_pos0(a, seg) + r;
  if (pos < a.keep[seg]) return;  // a ring cache no longer holds this position
  const int64_t src_row = (int64_t)a.row0[seg] + r;
  const int d = a.lay.d;
  const int block = a.table[(int64_t)a.seq[seg] * a.max_bps + (pos >> 8)];
  const int slot = pos & 255;
  uint8_t* base = a.pool + (int64_t)block * a.lay.block_bytes;
  T* kdst = reinterpret_cast<T*>(base + a.lay.k_off) + (int64_t)h * 256 * d;
  T* vdst = reinterpret_cast<T*>(base + a.lay.v_off) + (int64_t)h * 256 * d;
  const T* ksrc = reinterpret_cast<const T*>(a.k) + (src_row * a.lay.hkv + h) * d;
  const T* vsrc = reinterpret_cast<const T*>(a.v) + (src_row * a.lay.hkv + h) * d;
  for (int e = threadIdx.x; e < d; e += 64) {
    kdst[plain_k_index(FMT, d, slot, e)] = ksrc[e];
    vdst[plain_v_index(FMT, d, slot, e)] = vsrc[e];
  }
}

// ---- quantize-on-append ----------------------------------------------------------

// One workgroup (8 waves) per (segment, 32-token sub-tile, kv head).  Each
// wave encodes whole tokens (a decode step's <= 8 new rows: one each); key
// codes and scales go straight to their bytes (a byte never holds two
// tokens).  Value codes share 48-bit fields
// across 16 tokens, so they are staged in LDS and then merged into their
// fields by one thread each (one writer per field: no two workgroups race).
constexpr int kAppendWaves = 8;
// Rows of a sub-tile up to which keys and values are encoded on separate
// waves: 2 (kAppendWaves - n) >= n.
constexpr int kSplitRows = 2 * kAppendWaves / 3;
// Query vectors per wave in the rotation workgroups of the step launch.
constexpr int kQVec = 3;

// Shared memory of one TQ3 append workgroup.  S^T is staged in LDS once per
// workgroup for d <= 128 (64 KiB), so the projections of the key residuals
// and of the rotated queries read LDS instead of L2.
// A workgroup either encodes (residual and value-code buffers) or rotates
// queries (kQVec rotated vectors per wave), so the two share their LDS,
// which keeps two encoding workgroups per CU at d <= 128.
template <int D>
struct AppendTq3Smem {
  static constexpr bool kStage = D <= 128;
  struct Enc {
    double rbuf[kAppendWaves][D];
    uint8_t vcode[32][D];
  };
  union {
    Enc enc;
    float qbuf[kAppendWaves][kQVec * D];
  };
  float st_lds[kStage ? D * D : 4];
  uint32_t sat_any;
};
static_assert(sizeof(AppendTq3Smem<128>) <= 80 * 1024, "two encoding workgroups per CU");

// S^T into LDS in two steps, loads into registers and then stores, so that
// the loads can be issued ahead of work that does not need them: every
// thread holds NST 16-byte pieces in between.
template <int D>
struct StStage {
  static constexpr int NST = AppendTq3Smem<D>::kStage ? D * D / 4 / (kAppendWaves * 64) : 0;
  float4 r[NST > 0 ? NST : 1];
  __device__ __forceinline__ void load(const float* s_t) {
#pragma unroll
    for (int i = 0; i < NST; ++i) r[i] = reinterpret_cast<const float4*>(s_t)[threadIdx.x + i * kAppendWaves * 64];
  }
  __device__ __forceinline__ void store(float* st_lds) const {
#pragma unroll
    for (int i = 0; i < NST; ++i) reinterpret_cast<float4*>(st_lds)[threadIdx.x + i * kAppendWaves * 64] = r[i];
  }
};

template <int D>
__device__ __forceinline__ void append_tq3_block(const AppendArgs& a, int unit, int h, AppendTq3Smem<D>& sm) {
  constexpr int E = D / 64;
  constexpr int SB = tq3_sub_bytes(D);
  constexpr bool kStage = AppendTq3Smem<D>::kStage;
  static_assert(2 * D <= kAppendWaves * 64, "one value-code field pair per thread");
  auto& rbuf = sm.enc.rbuf;
  auto& vcode = sm.enc.vcode;
  float* st_lds = sm.st_lds;
  uint32_t& sat_any = sm.sat_any;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  // S^T first: its loads depend on nothing
  StStage<D> st;
  if constexpr (kStage) st.load(a.s_t);
  if (threadIdx.x == 0) sat_any = 0;
  const int seg = find_seg(a.unit0, a.n_segs, unit);
  const int pos0 = seg_pos0(a, seg);
  const int grp = (pos0 >> 5) + (unit - a.unit0[seg]);  // 32-token sub-tile of the sequence
  const int t0 = max(max(pos0, grp * 32), a.keep[seg]);  // ring caches store nothing below keep
  const int t1 = min(pos0 + a.n[seg], grp * 32 + 32);
  if (t0 >= t1) return;  // a spare unit, or one a ring cache drops (whole workgroup)
  const int nr = t1 - t0;
  // this wave's first source vector (see the assignment below), requested
  // before the block-table read
  SrcVec<D> first;
  {
    int t = -1;
    const void* base = a.k;
    if (nr <= kSplitRows) {
      if (wave < nr) {
        t = t0 + wave;
      } else if (wave - nr < nr) {
        t = t0 + wave - nr;
        base = a.v;
      }
    } else if (wave < 2 * nr) {
      const bool is_key = wave < nr;
      t = t0 + (is_key ? wave : wave - nr);
      base = is_key ? a.k : a.v;
    }
    if (t >= 0) {
      const int64_t src_row = (int64_t)a.row0[seg] + (t - pos0);
      first.load(reinterpret_cast<const float*>(base) + (src_row * a.lay.hkv + h) * D);
    }
  }
  const int block = a.table[(int64_t)a.seq[seg] * a.max_bps + (grp >> 3)];
  uint8_t* sub = a.pool + (int64_t)block * a.lay.block_bytes + ((int64_t)h * 8 + (grp & 7)) * SB;
  // The stored value-code fields this workgroup merges into (one thread per
  // (dimension, half): the 48-bit field of dimension i for the tokens with
  // bit 2 = half), read now so that the reads overlap the encoding.  Only
  // this workgroup writes this sub-tile's fields.
  const int fi = threadIdx.x >> 1, fsel = threadIdx.x & 1;
  uint8_t* fp = nullptr;
  uint64_t field = 0;
  if (threadIdx.x < 2 * D) {
    int bit0;
    fp = sub + tq3_v_field(D, 4 * fsel, fi, &bit0);  // any token of this half names the field
#pragma unroll
    for (int b = 0; b < 6; ++b) field |= (uint64_t)fp[b] << (8 * b);
  }
  if constexpr (kStage) st.store(st_lds);
  const float* s_t = kStage ? st_lds : a.s_t;
  uint32_t sat = 0;
  __syncthreads();
  // one wave per encoded vector.  Up to five rows (every value wave then
  // has at most two values, and a key costs about two values: its residual
  // projection): the keys of rows t0 + w on waves w < nr, the values on the
  // other waves, round robin; more rows: keys, then values, round robin
  // over all waves.
  auto enc_key = [&](int t, const SrcVec<D>& xs) {
    const int m = t & 31;
    EncOut<D> ko;
    encode_vector<D>(xs, true, a.signs, s_t, a.thr, a.lev16, rbuf[wave], ko, &sat);
    // key nibbles: dims 2b, 2b+1 share a byte
    if constexpr (E == 1) {
      const uint32_t nib = (uint32_t)(ko.code[0] | (ko.bit[0] << 3));
      const uint32_t hi = __shfl_down(nib, 1);
      if ((lane & 1) == 0) {
        int nb;
        sub[tq3_k_byte(D, m, lane, &nb)] = (uint8_t)(nib | (hi << 4));
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; e += 2) {
        const uint32_t lo = ko.code[e] | (ko.bit[e] << 3);
        const uint32_t hi = ko.code[e + 1] | (ko.bit[e + 1] << 3);
        int nb;
        sub[tq3_k_byte(D, m, lane * E + e, &nb)] = (uint8_t)(lo | (hi << 4));
      }
    }
    if (lane == 0) {
      store_half(sub + tq3_scale_byte(D, m, 0), ko.n16);
      store_half(sub + tq3_scale_byte(D, m, 1), ko.g16);
    }
  };
  auto enc_value = [&](int t, const SrcVec<D>& xs) {
    const int m = t & 31;
    EncOut<D> vo;
    encode_vector<D>(xs, false, a.signs, s_t, a.thr, a.lev16, rbuf[wave], vo, &sat);
#pragma unroll
    for (int e = 0; e < E; ++e) vcode[m][lane * E + e] = vo.code[e];
    if (lane == 0) store_half(sub + tq3_scale_byte(D, m, 2), vo.n16);
  };
  auto src_of = [&](const void* base, int t) {
    const int64_t src_row = (int64_t)a.row0[seg] + (t - pos0);
    return reinterpret_cast<const float*>(base) + (src_row * a.lay.hkv + h) * D;
  };
  if (nr <= kSplitRows) {
    if (wave < nr) {
      enc_key(t0 + wave, first);
    } else {
      bool have = true;
      for (int j = wave - nr; j < nr; j += kAppendWaves - nr) {
        SrcVec<D> xs;
        if (have)
          xs = first;
        else
          xs.load(src_of(a.v, t0 + j));
        have = false;
        enc_value(t0 + j, xs);
      }
    }
  } else {
    for (int it = wave; it < 2 * nr; it += kAppendWaves) {
      const bool is_key = it < nr;
      const int t = t0 + (is_key ? it : it - nr);
      SrcVec<D> xs;
      if (it == wave)
        xs = first;
      else
        xs.load(src_of(is_key ? a.k : a.v, t));
      if (is_key)
        enc_key(t, xs);
      else
        enc_value(t, xs);
    }
  }
  if (sat) atomicOr(&sat_any, 1u);
  __syncthreads();
  // Merge the staged value codes into their fields.
  const int m0 = t0 & 31, m1 = m0 + nr;
  if (threadIdx.x < 2 * D) {
    for (int m = m0; m < m1; ++m) {
      if (((m >> 2) & 1) != fsel) continue;
      int bit;
      tq3_v_field(D, m, fi, &bit);
      field = (field & ~((uint64_t)7 << bit)) | ((uint64_t)vcode[m][fi] << bit);
    }
#pragma unroll
    for (int b = 0; b < 6; ++b) fp[b] = (uint8_t)(field >> (8 * b));
  }
  if (threadIdx.x == 0 && sat_any) atomicOr(a.status, 1u);
}

template <int D>
__global__ __launch_bounds__(kAppendWaves * 64) void append_tq3_kernel(AppendArgs a) {
  __shared__ __align__(16) AppendTq3Smem<D> sm;
  append_tq3_block<D>(a, blockIdx.x, blockIdx.y, sm);
}

// A decode step's two small launches of the compressed path in one: the
// first n_app workgroups encode the appended rows (workgroup b: unit b / hkv,
// kv head b % hkv), the rest rotate the queries, eight vectors per
// workgroup.  The two jobs touch disjoint memory and run side by side.
template <int D>
__global__ __launch_bounds__(kAppendWaves * 64) void append_tq3_qprep_kernel(AppendArgs a, QPrepArgs q,
                                                                            int32_t n_app) {
  __shared__ __align__(16) AppendTq3Smem<D> sm;
  const int b = blockIdx.x;
  if (b < n_app) {
    append_tq3_block<D>(a, b / a.lay.hkv, b % a.lay.hkv, sm);
    return;
  }
  // query rotation: S^T staged once, kQVec vectors per wave (their loads
  // issued alongside the staging)
  constexpr bool kStage = AppendTq3Smem<D>::kStage;
  constexpr int NV = kQVec;
  const int wave = threadIdx.x >> 6;
  const int64_t vec0 = ((int64_t)(b - n_app) * kAppendWaves + wave) * NV;
  QVecs<D, NV> qv;
  if constexpr (kStage) {
    StStage<D> st;
    st.load(q.s_t);
    qv.load(q, vec0);
    st.store(sm.st_lds);
    __syncthreads();
  } else {
    qv.load(q, vec0);
  }
  if (vec0 < q.n_vec) qprep_vectors<D, NV>(q, vec0, qv, kStage ? sm.st_lds : q.s_t, sm.qbuf[wave]);
}

hipError_t launch_append_qprep(const AppendArgs& a, const QPrepArgs& q, hipStream_t s) {
  if (a.lay.fmt != 2 || q.d != a.lay.d) return hipErrorInvalidValue;
  const int64_t n_app = (int64_t)a.total_units * a.lay.hkv;
  const int64_t per_wg = (int64_t)kAppendWaves * kQVec;
  const int64_t n_q = (q.n_vec + per_wg - 1) / per_wg;
  if (n_app + n_q <= 0) return hipSuccess;
  if (n_app + n_q > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)(n_app + n_q)), block(kAppendWaves * 64);
  switch (a.lay.d) {
    case 64:
      hipLaunchKernelGGL(append_tq3_qprep_kernel<64>, grid, block, 0, s, a, q, (int32_t)n_app);
      break;
    case 128:
      hipLaunchKernelGGL(append_tq3_qprep_kernel<128>, grid, block, 0, s, a, q, (int32_t)n_app);
      break;
    case 256:
      hipLaunchKernelGGL(append_tq3_qprep_kernel<256>, grid, block, 0, s, a, q, (int32_t)n_app);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.total_units <= 0) return hipSuccess;
  dim3 grid(a.total_units, a.lay.hkv);
  if (a.lay.fmt == 0) {
    hipLaunchKernelGGL((append_plain_kernel<float, 0>), grid, dim3(64), 0, s, a);
  } else if (a.lay.fmt == 1) {
    hipLaunchKernelGGL((append_plain_kernel<uint16_t, 1>), grid, dim3(64), 0, s, a);
  } else {
    switch (a.lay.d) {
      case 64:
        hipLaunchKernelGGL(append_tq3_kernel<64>, grid, dim3(kAppendWaves * 64), 0, s, a);
        break;
      case 128:
        hipLaunchKernelGGL(append_tq3_kernel<128>, grid, dim3(kAppendWaves * 64), 0, s, a);
        break;
      case 256:
        hipLaunchKernelGGL(append_tq3_kernel<256>, grid, dim3(kAppendWaves * 64), 0, s, a);
        break;
      default:
        return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

// ---- stand-alone encode ------------------------------------------------------------

// One wave per vector, 4 vectors per workgroup.  Record layout: key = D/2
// nibble bytes, n16, g16; value = 3D/8 bytes of 3-bit codes (dim i at bits
// 3i..3i+2), n16.
template <int D>
__global__ __launch_bounds__(256) void encode_kernel(EncodeArgs a) {
  constexpr int E = D / 64;
  __shared__ double rbuf[4][D];
  __shared__ uint8_t codes[4][D];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t vec = (int64_t)blockIdx.x * 4 + wave;
  uint32_t sat = 0;
  if (vec < a.n) {
    const int rec = a.is_key ? (D / 2 + 4) : (3 * D / 8 + 2);
    uint8_t* dst = a.dst + vec * rec;
    EncOut<D> o;
    SrcVec<D> xs;
    xs.load(a.src + vec * D);
    encode_vector<D>(xs, a.is_key != 0, a.signs, a.s_t, a.thr, a.lev16, rbuf[wave], o, &sat);
    if (a.is_key) {
      store_key_nibbles<D>(dst, o);
      if (lane == 0) {
        store_half(dst + D / 2, o.n16);
        store_half(dst + D / 2 + 2, o.g16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) codes[wave][lane * E + e] = o.code[e];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int b = lane; b < 3 * D / 8; b += 64) {
        uint32_t val = 0;
        const int first = (8 * b) / 3, last = (8 * b + 7) / 3;
        for (int i = first; i <= last && i < D; ++i) {
          const int pos = 3 * i - 8 * b;  // bit of code i relative to byte b
          const uint32_t c = codes[wave][i];
          val |= pos >= 0 ? (c << pos) : (c >> (-pos));
        }
        dst[b] = (uint8_t)(val & 0xFF);
      }
      if (lane == 0) store_half(dst + 3 * D / 8, o.n16);
    }
    if (sat && lane == 0) atomicOr(a.status, 1u);
  }
}

hipError_t launch_encode(const EncodeArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  dim3 grid((unsigned)((a.n + 3) / 4));
  switch (a.d) {
    case 64:
      hipLaunchKernelGGL(encode_kernel<64>, grid, dim3(256), 0, s, a);
      break;
    case 128:
      hipLaunchKernelGGL(encode_kernel<128>, grid, dim3(256), 0, s, a);
      break;
    case 256:
      hipLaunchKernelGGL(encode_kernel<256>, grid, dim3(256), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace svattn
