// Device-side helpers shared by the gfx950 kernels of the MoE forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// Native 128-bit vector (HIP's uint4 is a struct; selects on it go through
// memory).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 storage is handled as raw 16-bit patterns.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even; inputs here are finite.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// The same rounding by gfx950's v_cvt_pk_bf16_f32 (one instruction, the
// same bits for finite inputs).  Used only where it was measured to help:
// in the grouped GEMM's dH / dX epilogue it made the compiler spill
// registers (that kernel 60% slower).
__device__ __forceinline__ uint16_t f32_to_bf16_hw(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) |
         (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Low / high bf16 of a 32-bit word, widened to fp32.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Cross-lane reductions by DPP: within each row of 16 lanes (quad swaps,
// then rotations by 4 and by 8 lanes), then the four row results, read from
// lanes 0, 16, 32 and 48 into scalar registers, combined in a fixed order;
// every lane gets the result.  Every lane must be active.
template <int Ctrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), Ctrl, 0xF, 0xF, false));
}

template <int Ctrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<Ctrl>(__float_as_uint(v)));
}

constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowRor4 = 0x124, kDppRowRor8 = 0x128;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppQuadXor1>(v));
  v = max(v, dpp_u32<kDppQuadXor2>(v));
  v = max(v, dpp_u32<kDppRowRor4>(v));
  v = max(v, dpp_u32<kDppRowRor8>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor4>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor8>(v));
  const float r0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float r1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  const float r2 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32));
  const float r3 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The row sums are those of lanes 0, 16, 32, 48, so the order of the adds
// is fixed: ((row 0 + row 1) + (row 2 + row 3)).
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowRor4>(v);
  v += dpp_f32<kDppRowRor8>(v);
  const float r0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float r1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  const float r2 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32));
  const float r3 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Total order on fp32 as unsigned keys (no NaNs expected).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace moe
