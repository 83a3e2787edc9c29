// Cross-row lane exchanges of a wave (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rskv {

// The value v holds in lane l ^ X, X = 16 or 32: what __shfl_xor(v, X)
// returns, from gfx950's row-swap permutes (v_permlane16_swap and
// v_permlane32_swap exchange 16-lane rows, resp. 32-lane halves, of two
// registers) instead of an LDS permute.  Swapping v with itself leaves the
// partner's value in the first result on lanes with bit X set and in the
// second result on the others.  Blocks are one-dimensional, so bit X of
// threadIdx.x is bit X of the lane index.
template <int X>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v) {
  static_assert(X == 16 || X == 32, "row swaps exchange 16 or 32 lanes");
  const auto r = X == 16 ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                         : __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & X) ? r[0] : r[1];
}
template <int X>
__device__ __forceinline__ float xor_lane(float v) {
  return __uint_as_float(xor_lane_u32<X>(__float_as_uint(v)));
}
template <int X>
__device__ __forceinline__ double xor_lane(double v) {
  const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(v));
  const uint32_t lo = xor_lane_u32<X>(static_cast<uint32_t>(u));
  const uint32_t hi = xor_lane_u32<X>(static_cast<uint32_t>(u >> 32));
  return __longlong_as_double(
      static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

}  // namespace rskv
