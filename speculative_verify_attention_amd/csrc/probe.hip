// probe.hip - streaming-read probe: the read bandwidth a single pass over a
// buffer reaches on this GPU, as a ceiling to compare the attention kernels'
// effective bandwidth with.  The words read are xor-folded so that no load
// is dead.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace svattn {

typedef uint32_t pu32x4_t __attribute__((ext_vector_type(4)));

// One workgroup per compute unit walks the buffer grid-stride: each step
// reads UNROLL wave-wide 1 KiB pieces per wave, kProbeWorkgroups x 4 KiB
// apart, so that all 256 compute units stream side by side through the
// whole buffer, with non-temporal loads (read once, as the attention
// kernels read the cache).  Measured over 2 GiB on MI355X (best of ten):
// this shape 6.5 TB/s with plain loads and 7.2 TB/s non-temporal; 512 to
// 4096 workgroups of 256 to 1024 threads, or contiguous chunks per
// workgroup, 5.3 to 6.4 TB/s.
template <int UNROLL>
__global__ __launch_bounds__(256) void stream_probe_kernel(const pu32x4_t* __restrict__ src, int64_t n16,
                                                           uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  pu32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    pu32x4_t x[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) x[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= x[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  uint32_t w = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) w ^= __shfl_xor(w, o);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

hipError_t launch_stream_probe(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  hipLaunchKernelGGL(stream_probe_kernel<16>, dim3(kProbeWorkgroups), dim3(256), 0, s,
                     static_cast<const pu32x4_t*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace svattn
