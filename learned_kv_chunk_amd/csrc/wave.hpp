// wave.hpp -- wave64 cross-lane primitives for gfx950 that stay in the VALU
// (DPP row operations, v_permlane16_swap / v_permlane32_swap, v_readlane)
// instead of routing data through the LDS crossbar (ds_bpermute).
//
// Lane layout facts these rely on (checked on the hardware):
//  * permlane16_swap(a, b) exchanges the odd 16-lane rows of `a` with the
//    even rows of `b`; with a == b == v the two results hold, in every lane,
//    v from the lane's own row pair {0,1} or {2,3}: combining them is an
//    xor-16 butterfly step.
//  * permlane32_swap(a, b) exchanges lanes 32..63 of `a` with lanes 0..31 of
//    `b`; with a == b == v combining the results is an xor-32 step.
//  * DPP row_shr:n with bound_ctrl moves lane i-n to lane i within each row
//    of 16 and writes 0 where i-n leaves the row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowMirror = 0x140;      // lane i of a row of 16 reads lane 15 - i
constexpr int kDppRowHalfMirror = 0x141;  // lane i of a row of 8 reads lane 7 - i
template <int N>
constexpr int dpp_row_shr() { return 0x110 + N; }

__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ uint32_t xor16_sum_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return r[0] + r[1];
}
__device__ __forceinline__ uint32_t xor32_sum_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return r[0] + r[1];
}

// Maximum over the 64 lanes, returned in every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor4>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor8>(v));
  return xor32_max(xor16_max(v));
}

// Sum over the 64 lanes, returned in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowRor4>(v);
  v += dpp_f32<kDppRowRor8>(v);
  return xor32_sum(xor16_sum(v));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_u32<kDppQuadXor1>(v);
  v += dpp_u32<kDppQuadXor2>(v);
  v += dpp_u32<kDppRowRor4>(v);
  v += dpp_u32<kDppRowRor8>(v);
  return xor32_sum_u32(xor16_sum_u32(v));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppQuadXor1>(v));
  v = max(v, dpp_u32<kDppQuadXor2>(v));
  v = max(v, dpp_u32<kDppRowRor4>(v));
  v = max(v, dpp_u32<kDppRowRor8>(v));
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(r[0], r[1]);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<kDppQuadXor1>(v));
  v = min(v, dpp_u32<kDppQuadXor2>(v));
  v = min(v, dpp_u32<kDppRowRor4>(v));
  v = min(v, dpp_u32<kDppRowRor8>(v));
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min(r[0], r[1]);
}

// Sum over each aligned group of G lanes (G = 4, 8, 16 or 32), returned in
// every lane of the group: xor-1 and xor-2 steps inside quads, then the
// mirrored half-row (the other quad of 8 lanes), the mirrored row (the other
// 8 lanes of 16) and the xor-16 swap.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 4 || G == 8 || G == 16 || G == 32, "group of 4, 8, 16 or 32 lanes");
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  if constexpr (G >= 8) v += dpp_f32<kDppRowHalfMirror>(v);
  if constexpr (G >= 16) v += dpp_f32<kDppRowMirror>(v);
  if constexpr (G >= 32) v = xor16_sum(v);
  return v;
}

// Inclusive prefix sum over lanes 0..63 (lane i gets sum of lanes 0..i).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += dpp_u32<dpp_row_shr<1>()>(v);
  v += dpp_u32<dpp_row_shr<2>()>(v);
  v += dpp_u32<dpp_row_shr<4>()>(v);
  v += dpp_u32<dpp_row_shr<8>()>(v);
  const uint32_t t0 = __builtin_amdgcn_readlane(v, 15);
  const uint32_t t1 = __builtin_amdgcn_readlane(v, 31);
  const uint32_t t2 = __builtin_amdgcn_readlane(v, 47);
  const uint32_t row = (threadIdx.x & 63u) >> 4;
  v += (row > 0 ? t0 : 0u) + (row > 1 ? t1 : 0u) + (row > 2 ? t2 : 0u);
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const uint32_t lane = threadIdx.x & 63u;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace lsa
