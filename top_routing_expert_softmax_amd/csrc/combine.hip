// Weighted combine back to token order: "CMU 11-868 Lecture 17" section 2.2
// (add the expert outputs back with their weights) and "MoE routing math"
// section 2.2 (shared experts added with weight 1).
//
// One wavefront per token; lanes walk the d dimension in 16-byte chunks, so
// every load and store is coalesced.  fp32 accumulation, shared experts
// first, then j = 0..k-1; a dropped pair (row -1) adds nothing.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxK = 64;
constexpr int kTokPB = 4;   // tokens (wavefronts) per block

__device__ __forceinline__ void acc_chunk(float (&a)[8], const uint4 q, float w) {
  a[0] = fmaf(w, bf16lo(q.x), a[0]); a[1] = fmaf(w, bf16hi(q.x), a[1]);
  a[2] = fmaf(w, bf16lo(q.y), a[2]); a[3] = fmaf(w, bf16hi(q.y), a[3]);
  a[4] = fmaf(w, bf16lo(q.z), a[4]); a[5] = fmaf(w, bf16hi(q.z), a[5]);
  a[6] = fmaf(w, bf16lo(q.w), a[6]); a[7] = fmaf(w, bf16hi(q.w), a[7]);
}

// bf16: a chunk is 8 values (uint4).
__global__ __launch_bounds__(256) void combine_bf16_kernel(
    const uint4* __restrict__ y_perm, const uint4* __restrict__ y_shared,
    const int32_t* __restrict__ row_of_pair, const float* __restrict__ topk_w,
    uint4* __restrict__ y, int nT, int k, int E_shared, int chunks) {
  __shared__ int s_rows[kTokPB][kMaxK];
  __shared__ float s_w[kTokPB][kMaxK];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int t = blockIdx.x * kTokPB + wv;
  if (t >= nT) return;
  if (lane < k) {
    s_rows[wv][lane] = row_of_pair[static_cast<int64_t>(t) * k + lane];
    s_w[wv][lane] = topk_w[static_cast<int64_t>(t) * k + lane];
  }
  __builtin_amdgcn_wave_barrier();
  const int* rows = s_rows[wv];
  const float* ws = s_w[wv];
  for (int c = lane; c < chunks; c += kWave) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < E_shared; ++s)
      acc_chunk(a, y_shared[(static_cast<int64_t>(s) * nT + t) * chunks + c], 1.0f);
    for (int j = 0; j < k; ++j)
      if (rows[j] >= 0) acc_chunk(a, y_perm[static_cast<int64_t>(rows[j]) * chunks + c], ws[j]);
    uint4 o;
    o.x = pack_bf16x2(a[0], a[1]);
    o.y = pack_bf16x2(a[2], a[3]);
    o.z = pack_bf16x2(a[4], a[5]);
    o.w = pack_bf16x2(a[6], a[7]);
    y[static_cast<int64_t>(t) * chunks + c] = o;
  }
}

// fp32: a chunk is 4 values (float4).
__global__ __launch_bounds__(256) void combine_f32_kernel(
    const float4* __restrict__ y_perm, const float4* __restrict__ y_shared,
    const int32_t* __restrict__ row_of_pair, const float* __restrict__ topk_w,
    float4* __restrict__ y, int nT, int k, int E_shared, int chunks) {
  __shared__ int s_rows[kTokPB][kMaxK];
  __shared__ float s_w[kTokPB][kMaxK];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int t = blockIdx.x * kTokPB + wv;
  if (t >= nT) return;
  if (lane < k) {
    s_rows[wv][lane] = row_of_pair[static_cast<int64_t>(t) * k + lane];
    s_w[wv][lane] = topk_w[static_cast<int64_t>(t) * k + lane];
  }
  __builtin_amdgcn_wave_barrier();
  const int* rows = s_rows[wv];
  const float* ws = s_w[wv];
  for (int c = lane; c < chunks; c += kWave) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < E_shared; ++s) {
      const float4 q = y_shared[(static_cast<int64_t>(s) * nT + t) * chunks + c];
      a.x += q.x; a.y += q.y; a.z += q.z; a.w += q.w;
    }
    for (int j = 0; j < k; ++j) {
      if (rows[j] < 0) continue;
      const float4 q = y_perm[static_cast<int64_t>(rows[j]) * chunks + c];
      a.x = fmaf(ws[j], q.x, a.x); a.y = fmaf(ws[j], q.y, a.y);
      a.z = fmaf(ws[j], q.z, a.z); a.w = fmaf(ws[j], q.w, a.w);
    }
    y[static_cast<int64_t>(t) * chunks + c] = a;
  }
}

}  // namespace

hipError_t launch_combine(int64_t T, int64_t d, int E_shared, int k, bool bf16,
                          const void* y_perm, const void* y_shared,
                          const int32_t* row_of_pair, const float* topk_w, void* y,
                          hipStream_t s) {
  const int tokens_per_block = kTokPB;
  const dim3 grid(static_cast<unsigned>((T + tokens_per_block - 1) / tokens_per_block));
  const dim3 block(tokens_per_block * kWave);
  if (bf16) {
    hipLaunchKernelGGL(combine_bf16_kernel, grid, block, 0, s,
                       static_cast<const uint4*>(y_perm), static_cast<const uint4*>(y_shared),
                       row_of_pair, topk_w, static_cast<uint4*>(y), static_cast<int>(T), k,
                       E_shared, static_cast<int>(d / 8));
  } else {
    hipLaunchKernelGGL(combine_f32_kernel, grid, block, 0, s,
                       static_cast<const float4*>(y_perm), static_cast<const float4*>(y_shared),
                       row_of_pair, topk_w, static_cast<float4*>(y), static_cast<int>(T), k,
                       E_shared, static_cast<int>(d / 4));
  }
  return hipGetLastError();
}

}  // namespace moe
