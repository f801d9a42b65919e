// gdn_lane.hpp -- cross-lane sums within a wave (DPP) and 16-element row loads,
// for the kernels that keep one state column on a lane quad.
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

namespace gdn {
namespace lane {

// x + (x of the lane selected by DPP control `ctrl`).
template <int ctrl>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xb1, kQuadXor2 = 0x4e;  // quad_perm [1,0,3,2] and [2,3,0,1]
constexpr int kRowRor4 = 0x124, kRowRor8 = 0x128;  // row_ror:4 and row_ror:8

// Sum over the lane quad (the four row quarters of a column), in every lane of it.
__device__ __forceinline__ float quad_sum(float x) { return dpp_add<kQuadXor2>(dpp_add<kQuadXor1>(x)); }

// Sum over the wave (uniform result).
__device__ __forceinline__ float wave_sum(float x) {
  x = dpp_add<kRowRor8>(dpp_add<kRowRor4>(quad_sum(x)));  // every lane: the sum of its row of 16
  const int xi = __builtin_bit_cast(int, x);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48)));
}

typedef __attribute__((ext_vector_type(4))) unsigned int u32v4;
typedef __attribute__((ext_vector_type(4))) float f32v4;

// 16 consecutive elements from p (16-byte aligned), as stored.
template <class IT> struct Row;
template <> struct Row<float> {
  f32v4 w[4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = reinterpret_cast<const f32v4*>(p)[i];
  }
  __device__ __forceinline__ float operator[](int i) const { return w[i / 4][i % 4]; }
};
template <> struct Row<__hip_bfloat16> {
  u32v4 w[2];
  __device__ __forceinline__ void load(const __hip_bfloat16* p) {
#pragma unroll
    for (int i = 0; i < 2; ++i) w[i] = reinterpret_cast<const u32v4*>(p)[i];
  }
  __device__ __forceinline__ float operator[](int i) const {
    const unsigned x = w[i / 8][(i % 8) / 2];
    return __builtin_bit_cast(float, (i % 2) ? (x & 0xffff0000u) : (x << 16));
  }
};

}  // namespace lane
}  // namespace gdn
