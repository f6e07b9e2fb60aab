// Weighted combine back to token order: "CMU 11-868 Lecture 17" section 2.2
// (add the expert outputs back with their weights) and "MoE routing math"
// section 2.2 (shared experts added with weight 1).
//
// One wavefront per token (per slice of the row when there are few tokens);
// lanes walk the d dimension in 16-byte chunks, so every load and store is
// coalesced.  fp32 accumulation, shared experts first, then j = 0..k-1; a
// dropped pair (row -1) adds nothing.
#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxK = 256;   // k; expert choice passes k = E
constexpr int kTokPB = 4;   // tokens (wavefronts) per block

__device__ __forceinline__ void acc_chunk(float (&a)[8], const u32x4_t q, float w) {
  a[0] = fmaf(w, bf16lo(q.x), a[0]); a[1] = fmaf(w, bf16hi(q.x), a[1]);
  a[2] = fmaf(w, bf16lo(q.y), a[2]); a[3] = fmaf(w, bf16hi(q.y), a[3]);
  a[4] = fmaf(w, bf16lo(q.z), a[4]); a[5] = fmaf(w, bf16hi(q.z), a[5]);
  a[6] = fmaf(w, bf16lo(q.w), a[6]); a[7] = fmaf(w, bf16hi(q.w), a[7]);
}

// bf16: a chunk is 8 values (16 bytes).  blockIdx.y picks a slice of
// kWave chunks of the row (several slices when there are few tokens, so
// the chip has enough wavefronts); each lane's loads of the k expert rows
// are issued in groups of eight before they are summed, in order.
__global__ __launch_bounds__(256) void combine_bf16_kernel(
    const u32x4_t* __restrict__ y_perm, const u32x4_t* __restrict__ y_shared,
    const int32_t* __restrict__ row_of_pair, const float* __restrict__ topk_w,
    u32x4_t* __restrict__ y, int nT, int k, int E_shared, int chunks) {
  __shared__ int s_rows[kTokPB][kMaxK];
  __shared__ float s_w[kTokPB][kMaxK];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int t = blockIdx.x * kTokPB + wv;
  if (t >= nT) return;
  for (int j = lane; j < k; j += kWave) {
    s_rows[wv][j] = row_of_pair[static_cast<int64_t>(t) * k + j];
    s_w[wv][j] = topk_w[static_cast<int64_t>(t) * k + j];
  }
  __builtin_amdgcn_wave_barrier();
  const int* rows = s_rows[wv];
  const float* ws = s_w[wv];
  const int cstep = kWave * gridDim.y;
  for (int c = blockIdx.y * kWave + lane; c < chunks; c += cstep) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < E_shared; ++s)
      acc_chunk(a, y_shared[(static_cast<int64_t>(s) * nT + t) * chunks + c], 1.0f);
    for (int j0 = 0; j0 < k; j0 += 8) {
      u32x4_t q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        const int r = j < k ? rows[j] : -1;
        // r is the same for the whole wavefront (one token): no divergence
        q[u] = r >= 0 ? y_perm[static_cast<int64_t>(r) * chunks + c] : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        if (j < k && rows[j] >= 0) acc_chunk(a, q[u], ws[j]);
      }
    }
    u32x4_t o;
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
  for (int j = lane; j < k; j += kWave) {
    s_rows[wv][j] = row_of_pair[static_cast<int64_t>(t) * k + j];
    s_w[wv][j] = topk_w[static_cast<int64_t>(t) * k + j];
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
  const dim3 block(tokens_per_block * kWave);
  if (bf16) {
    // few tokens: split each row into up to chunks/kWave slices so that
    // about 2048 wavefronts run
    const int64_t chunks = d / 8;
    const int64_t max_slices = (chunks + kWave - 1) / kWave;
    const int64_t slices = std::max<int64_t>(1, std::min<int64_t>(max_slices, (2048 + T - 1) / T));
    const dim3 grid(static_cast<unsigned>((T + tokens_per_block - 1) / tokens_per_block),
                    static_cast<unsigned>(slices));
    hipLaunchKernelGGL(combine_bf16_kernel, grid, block, 0, s,
                       static_cast<const u32x4_t*>(y_perm), static_cast<const u32x4_t*>(y_shared),
                       row_of_pair, topk_w, static_cast<u32x4_t*>(y), static_cast<int>(T), k,
                       E_shared, static_cast<int>(chunks));
  } else {
    const dim3 grid(static_cast<unsigned>((T + tokens_per_block - 1) / tokens_per_block));
    hipLaunchKernelGGL(combine_f32_kernel, grid, block, 0, s,
                       static_cast<const float4*>(y_perm), static_cast<const float4*>(y_shared),
                       row_of_pair, topk_w, static_cast<float4*>(y), static_cast<int>(T), k,
                       E_shared, static_cast<int>(d / 4));
  }
  return hipGetLastError();
}

}  // namespace moe
