// lanes.h - the value of lane l ^ HL of a wavefront, without an LDS round
// trip: DPP moves within 16-lane rows (HL = 1, 2, 4, 8) and the gfx950 lane
// swaps across rows (HL = 16, 32).  Each returns exactly the partner lane's
// bits, so reductions and butterflies written with them compute what the
// same code with a shuffle through LDS computes, bit for bit.  Every lane
// of the wave must be active.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace svattn {

template <int HL>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t u) {
  static_assert(HL == 1 || HL == 2 || HL == 4 || HL == 8 || HL == 16 || HL == 32, "partner distance");
  const int x = (int)u;
  if constexpr (HL == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  } else if constexpr (HL == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  } else if constexpr (HL == 4) {
    // half-row mirror (q -> 7 - q in each group of 8), then quad reverse
    // (q -> q ^ 3): 7 - (q ^ 3) = q ^ 4
    const int y = __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false);
    return (uint32_t)__builtin_amdgcn_update_dpp(y, y, 0x1B, 0xF, 0xF, false);
  } else if constexpr (HL == 8) {
    return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false);  // row_ror 8
  } else if constexpr (HL == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}

template <int HL>
__device__ __forceinline__ float lane_xor(float v) {
  return __builtin_bit_cast(float, lane_xor_u32<HL>(__builtin_bit_cast(uint32_t, v)));
}

template <int HL>
__device__ __forceinline__ double lane_xor(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = lane_xor_u32<HL>((uint32_t)b), hi = lane_xor_u32<HL>((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, lo | (hi << 32));
}

// The value of lane j (wave-uniform j), bit for bit.
__device__ __forceinline__ float lane_value(float v, int j) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
}

// One butterfly stage of a Walsh-Hadamard transform across the wave: the
// lane with bit HL clear keeps v + partner, the other partner - v.
template <int HL, typename T, int E>
__device__ __forceinline__ void wht_stage(T (&v)[E], int lane) {
  const bool upper = (lane & HL) != 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const T p = lane_xor<HL>(v[e]);
    v[e] = upper ? (p - v[e]) : (v[e] + p);
  }
}

// The six cross-lane stages, partner distances 1, 2, 4, ..., 32.
template <typename T, int E>
__device__ __forceinline__ void wht_lanes(T (&v)[E], int lane) {
  wht_stage<1>(v, lane);
  wht_stage<2>(v, lane);
  wht_stage<4>(v, lane);
  wht_stage<8>(v, lane);
  wht_stage<16>(v, lane);
  wht_stage<32>(v, lane);
}

// Sum over the wave in the order 32, 16, 8, 4, 2, 1 (every lane gets it).
template <typename T>
__device__ __forceinline__ T lanes_sum(T v) {
  v += lane_xor<32>(v);
  v += lane_xor<16>(v);
  v += lane_xor<8>(v);
  v += lane_xor<4>(v);
  v += lane_xor<2>(v);
  v += lane_xor<1>(v);
  return v;
}

}  // namespace svattn
