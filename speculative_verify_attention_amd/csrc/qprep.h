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
#pragma unroll
  for (int hl = 1; hl < 64; hl <<= 1) {
    const bool upper = (lane & hl) != 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float p = __shfl_xor(v[e], hl);
      v[e] = upper ? (p - v[e]) : (v[e] + p);
    }
  }
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

}  // namespace svattn
