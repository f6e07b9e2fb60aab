// Per-row FP8 quantisation of expert weights: OCP E4M3 codes with one fp32
// scale per stored row (the pages name FP8 expert storage, "CMU 11-868
// Lecture 17" section 1.4, but no encoding).  For a row w:
//   s = max|w| / 448 (fp32 division, correctly rounded; 1 for an all-zero
//       row), code_i = E4M3 round-to-nearest-even of fp32(w_i / s), with
//       magnitudes clamped to 448, the largest finite E4M3 value.
// The rounding is written out in integer and exact fp32 operations, so the
// codes do not depend on a conversion instruction's rounding or saturation.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

// E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 holds
// the subnormals m * 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fminf(fabsf(q), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                                   // below 2^-6: grid 2^-9
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));   // 0..8; 8 is 2^-6
  } else {
    const uint32_t bits = __float_as_uint(a);
    int E = static_cast<int>((bits >> 23) & 0xFFu) - 127;         // 2^E <= a < 2^(E+1)
    const float mant = __uint_as_float((bits & 0x007FFFFFu) | 0x3F800000u);   // [1, 2)
    uint32_t n = static_cast<uint32_t>(__builtin_rintf(mant * 8.0f));       // 8..16
    if (n == 16u) { ++E; n = 8u; }
    code = (static_cast<uint32_t>(E + 7) << 3) | (n - 8u);
  }
  return code | sign;
}

template <typename T>
__device__ __forceinline__ float load_w(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_w<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}
template <>
__device__ __forceinline__ float load_w<float>(const float* p, int64_t i) { return p[i]; }

// One block per row: the row maximum, then the codes.
template <typename T>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const T* __restrict__ w,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ scales,
                                                           int64_t cols) {
  __shared__ float wmax[256 / kWave];
  const int64_t row = blockIdx.x;
  const T* src = w + row * cols;
  uint8_t* dst = codes + row * cols;
  float m = 0.f;
  for (int64_t i = threadIdx.x; i < cols; i += blockDim.x) m = fmaxf(m, fabsf(load_w(src, i)));
  m = wave_max(m);
  if ((threadIdx.x & (kWave - 1)) == 0) wmax[threadIdx.x / kWave] = m;
  __syncthreads();
  float amax = wmax[0];
#pragma unroll
  for (int i = 1; i < 256 / kWave; ++i) amax = fmaxf(amax, wmax[i]);
  const float s = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  for (int64_t i = threadIdx.x; i < cols; i += blockDim.x)
    dst[i] = static_cast<uint8_t>(e4m3_rne(__fdiv_rn(load_w(src, i), s)));
  if (threadIdx.x == 0) scales[row] = s;
}

}  // namespace

hipError_t launch_quantize_fp8(int64_t rows, int64_t cols, bool bf16, const void* w,
                               uint8_t* codes, float* scales, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(quantize_fp8_kernel<uint16_t>, dim3(static_cast<unsigned>(rows)),
                       dim3(256), 0, s, static_cast<const uint16_t*>(w), codes, scales, cols);
  else
    hipLaunchKernelGGL(quantize_fp8_kernel<float>, dim3(static_cast<unsigned>(rows)), dim3(256),
                       0, s, static_cast<const float*>(w), codes, scales, cols);
  return hipGetLastError();
}

}  // namespace moe
