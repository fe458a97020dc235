// qprep.h - the query rotation of the compressed cache's verify path, one
// wave per query vector: q' = H (D q) / sqrt(d) with an in-register
// Walsh-Hadamard transform, then q'' = S q' (S read transposed, coalesced).
// Called by the rotation kernel and by the step launch that encodes the new
// rows and rotates the queries side by side.
//
// SwiftLM page, TurboQuant KV-cache compression passage: keys are stored
// rotated (and with a QJL sign residual), so the few queries are rotated
// once instead of the many keys being rotated back.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.h"
#include "lanes.h"

namespace svattn {

// wb: D floats of this wave's LDS.
template <int D>
__device__ __forceinline__ void qprep_vector(const QPrepArgs& a, int64_t vec, float* wb) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lane * E + e;
    const float x = a.q[vec * D + i];
    v[e] = a.signs[i] < 0 ? -x : x;
  }
#pragma unroll
  for (int h = 1; h < E; h <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (!(e & h)) {
        const float x = v[e], y = v[e + h];
        v[e] = x + y;
        v[e + h] = x - y;
      }
  wht_lanes(v, lane);
  const float inv = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v[e] *= inv;
    a.q1[vec * D + lane * E + e] = v[e];
    wb[lane * E + e] = v[e];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // four partial sums per output (rows j = u mod 4): four independent fma
  // chains, and the loop unrolled so that many rows of S^T are in flight
  float acc[4][E];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[u][e] = 0.0f;
#pragma unroll 4
  for (int j = 0; j < D; j += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float qj = wb[j + u];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[u][e] = fmaf(a.s_t[(j + u) * D + lane * E + e], qj, acc[u][e]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) a.q2[vec * D + lane * E + e] = (acc[0][e] + acc[1][e]) + (acc[2][e] + acc[3][e]);
}

// NV query vectors vec0 .. vec0 + NV - 1 (those below a.n_vec) on one wave,
// with S^T read from s_t (LDS or global): each element of S^T is read once
// for all NV vectors.  The same operations in the same order as
// qprep_vector, so the results are bitwise those of one vector at a time.
// wb: NV * D floats of this wave's LDS.
// The lane's values of NV query vectors (zero past a.n_vec), loaded ahead
// of the rotation so that the loads overlap other set-up work.
template <int D, int NV>
struct QVecs {
  float x[NV][D / 64];
  __device__ __forceinline__ void load(const QPrepArgs& a, int64_t vec0) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < NV; ++u)
#pragma unroll
      for (int e = 0; e < D / 64; ++e)
        x[u][e] = vec0 + u < a.n_vec ? a.q[(vec0 + u) * D + lane * (D / 64) + e] : 0.0f;
  }
};

template <int D, int NV>
__device__ __forceinline__ void qprep_vectors(const QPrepArgs& a, int64_t vec0, const QVecs<D, NV>& qv,
                                              const float* s_t, float* wb) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  float v[NV][E];
#pragma unroll
  for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = lane * E + e;
      v[u][e] = a.signs[i] < 0 ? -qv.x[u][e] : qv.x[u][e];
    }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
#pragma unroll
    for (int h = 1; h < E; h <<= 1)
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (!(e & h)) {
          const float x = v[u][e], y = v[u][e + h];
          v[u][e] = x + y;
          v[u][e + h] = x - y;
        }
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) wht_lanes(v[u], lane);
  const float inv = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      v[u][e] *= inv;
      if (vec0 + u < a.n_vec) a.q1[(vec0 + u) * D + lane * E + e] = v[u][e];
      wb[u * D + lane * E + e] = v[u][e];
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float acc[NV][4][E];
#pragma unroll
  for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[u][r][e] = 0.0f;
#pragma unroll 2
  for (int j = 0; j < D; j += 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float sv[E];
#pragma unroll
      for (int e = 0; e < E; ++e) sv[e] = s_t[(j + r) * D + lane * E + e];
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const float qj = wb[u * D + j + r];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[u][r][e] = fmaf(sv[e], qj, acc[u][r][e]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NV; ++u)
    if (vec0 + u < a.n_vec)
#pragma unroll
      for (int e = 0; e < E; ++e)
        a.q2[(vec0 + u) * D + lane * E + e] = (acc[u][0][e] + acc[u][1][e]) + (acc[u][2][e] + acc[u][3][e]);
}

}  // namespace svattn
