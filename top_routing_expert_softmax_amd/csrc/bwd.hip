// Backward of the combine and of the router (bf16 activations, fp32 math).
//
// With L = sum(dy * y) + alpha * L_balance + beta * z:
//   combine ("CMU 11-868 Lecture 17" section 2.2; "MoE routing math"
//   section 2.2):  dO_tj = p~_tj dy_t for a kept pair (the rows of the
//   expert backward), dp~_tj = <dy_t, o_tj>, 0 for a dropped pair; each
//   shared expert's output gradient is dy itself.
//   router ("MoE routing math" sections 2.1, 3.4; [SA] router_z_loss):
//   p~_t is the softmax of the token's selected logits, so
//     dg_tj += p~_tj (dp~_tj - sum_j' p~_tj' dp~_tj')   for j in S_t;
//   the balance loss reaches g only through P_i (f_i are counts):
//     dg_ti += p_ti (c_i - sum_i' p_ti' c_i'),  c_i = alpha E f_i / T;
//   the z-loss:  dg_ti += 2 beta lse_t p_ti / T.
//   dW_gate = x^T dg,  dx_t = sum_s dX_s,t + sum_j dX_tj + dg_t W_gate^T.
#include <math.h>

#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxKb = 64;

__device__ __forceinline__ void unpack8(const u32x4_t q, float (&v)[8]) {
  v[0] = bf16lo(q.x); v[1] = bf16hi(q.x); v[2] = bf16lo(q.y); v[3] = bf16hi(q.y);
  v[4] = bf16lo(q.z); v[5] = bf16hi(q.z); v[6] = bf16lo(q.w); v[7] = bf16hi(q.w);
}

__device__ __forceinline__ u32x4_t pack8(const float (&v)[8]) {
  u32x4_t o;
  o.x = pack_bf16x2(v[0], v[1]);
  o.y = pack_bf16x2(v[2], v[3]);
  o.z = pack_bf16x2(v[4], v[5]);
  o.w = pack_bf16x2(v[6], v[7]);
  return o;
}

// One wavefront per token; 16-byte chunks of d over the lanes.
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const u32x4_t* __restrict__ dy, const u32x4_t* __restrict__ y_perm,
    const int32_t* __restrict__ row_of_pair, const float* __restrict__ topk_w,
    u32x4_t* __restrict__ dy_perm, float* __restrict__ dtopk_w, int T, int k, int Es,
    int chunks) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const u32x4_t* dyt = dy + static_cast<int64_t>(t) * chunks;
  for (int j = 0; j < k; ++j) {
    const int r = row_of_pair[static_cast<int64_t>(t) * k + j];
    float dot = 0.f;
    if (r >= 0) {
      const float w = topk_w[static_cast<int64_t>(t) * k + j];
      for (int c = lane; c < chunks; c += kWave) {
        float g[8], o[8];
        unpack8(dyt[c], g);
        unpack8(y_perm[static_cast<int64_t>(r) * chunks + c], o);
#pragma unroll
        for (int u = 0; u < 8; ++u) dot = fmaf(g[u], o[u], dot);
        float s[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) s[u] = w * g[u];
        dy_perm[static_cast<int64_t>(r) * chunks + c] = pack8(s);
      }
    }
    dot = wave_sum(dot);
    if (lane == 0) dtopk_w[static_cast<int64_t>(t) * k + j] = dot;
  }
  for (int s = 0; s < Es; ++s) {
    u32x4_t* dst = dy_perm + (static_cast<int64_t>(T) * k + static_cast<int64_t>(s) * T + t) * chunks;
    for (int c = lane; c < chunks; c += kWave) dst[c] = dyt[c];
  }
}

// One wavefront per token: dg_t over the E experts (lane holds experts
// lane + 64 r).
__global__ __launch_bounds__(256) void route_dg_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const float* __restrict__ dtopk_w,
    const int32_t* __restrict__ counts, float* __restrict__ dg, int T, int E, int k,
    float alpha, float beta) {
  __shared__ float srow[256 / kWave][256];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int t = blockIdx.x * (blockDim.x / kWave) + wv;
  if (t >= T) return;
  const float* g = logits + static_cast<int64_t>(t) * E;
  float gv[4], m = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane + kWave * r;
    gv[r] = e < E ? g[e] : -INFINITY;
    m = fmaxf(m, gv[r]);
  }
  m = wave_max(m);
  float z = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) z += (lane + kWave * r < E) ? expf(gv[r] - m) : 0.f;
  z = wave_sum(z);
  const float lse = m + logf(z);
  const float invT = 1.0f / static_cast<float>(T);
  float p[4], c[4], pc = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane + kWave * r;
    p[r] = e < E ? expf(gv[r] - lse) : 0.f;
    c[r] = e < E ? alpha * static_cast<float>(E) * static_cast<float>(counts[e]) * invT * invT
                 : 0.f;
    pc += p[r] * c[r];
  }
  pc = wave_sum(pc);
  float* row = srow[wv];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane + kWave * r;
    if (e < E) row[e] = p[r] * (c[r] - pc) + 2.0f * beta * lse * p[r] * invT;
  }
  // selected experts: p~ (dp~ - <p~, dp~>), added by the lane that owns j
  float pw = 0.f;
  for (int j = lane; j < k; j += kWave)
    pw += topk_w[static_cast<int64_t>(t) * k + j] * dtopk_w[static_cast<int64_t>(t) * k + j];
  pw = wave_sum(pw);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int j = lane; j < k; j += kWave) {
    const int e = topk_idx[static_cast<int64_t>(t) * k + j];
    if (e >= 0 && e < E)
      row[e] += topk_w[static_cast<int64_t>(t) * k + j] *
                (dtopk_w[static_cast<int64_t>(t) * k + j] - pw);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int e = lane; e < E; e += kWave) dg[static_cast<int64_t>(t) * E + e] = row[e];
}

// dx_t = sum_s dx_shared[s][t] + sum_j dx_perm[row_of_pair[t][j]] +
// sum_e dg[t][e] W_gate[:, e], in that order; one wavefront per token.
__global__ __launch_bounds__(256) void dx_kernel(
    const u32x4_t* __restrict__ dx_perm, const u32x4_t* __restrict__ dx_shared,
    const int32_t* __restrict__ row_of_pair, const float* __restrict__ dg,
    const uint16_t* __restrict__ w_gate, u32x4_t* __restrict__ dx, int T, int E, int k, int Es,
    int chunks) {
  __shared__ float sdg[256 / kWave][256];
  __shared__ int srows[256 / kWave][kMaxKb];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int t = blockIdx.x * (blockDim.x / kWave) + wv;
  if (t >= T) return;
  for (int e = lane; e < E; e += kWave) sdg[wv][e] = dg[static_cast<int64_t>(t) * E + e];
  for (int j = lane; j < k; j += kWave) srows[wv][j] = row_of_pair[static_cast<int64_t>(t) * k + j];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int c = lane; c < chunks; c += kWave) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float v[8];
    for (int s = 0; s < Es; ++s) {
      unpack8(dx_shared[(static_cast<int64_t>(s) * T + t) * chunks + c], v);
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] += v[u];
    }
    for (int j = 0; j < k; ++j) {
      const int r = srows[wv][j];
      if (r < 0) continue;
      unpack8(dx_perm[static_cast<int64_t>(r) * chunks + c], v);
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] += v[u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint16_t* wrow = w_gate + static_cast<int64_t>(c * 8 + u) * E;
      float s = 0.f;
      if (E % 8 == 0) {
        // the row in 16-byte pieces (rows are 16-byte aligned), same order
        for (int q = 0; q < E / 8; ++q) {
          float w[8];
          unpack8(reinterpret_cast<const u32x4_t*>(wrow)[q], w);
#pragma unroll
          for (int v2 = 0; v2 < 8; ++v2) s = fmaf(sdg[wv][q * 8 + v2], w[v2], s);
        }
      } else {
        for (int e = 0; e < E; ++e) s = fmaf(sdg[wv][e], bf16_to_f32(wrow[e]), s);
      }
      a[u] += s;
    }
    dx[static_cast<int64_t>(t) * chunks + c] = pack8(a);
  }
}

// dw_gate[i][e] = sum_t x[t][i] dg[t][e] over the token slice blockIdx.z
// (t in order): thread i, experts e0 .. e0+7.  With several slices the
// partial sums go to part[slice] and dwgate_sum_kernel adds them in slice
// order, so the result does not depend on the schedule.
__global__ __launch_bounds__(256) void dwgate_kernel(const uint16_t* __restrict__ x,
                                                     const float* __restrict__ dg,
                                                     float* __restrict__ part, int T, int d,
                                                     int E, int chunk) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int e0 = blockIdx.y * 8;
  if (i >= d) return;
  const int t0 = blockIdx.z * chunk;
  const int t1 = min(T, t0 + chunk);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr int kU = 8;                          // x loads in flight per thread
  int t = t0;
  for (; t + kU <= t1; t += kU) {
    float xv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) xv[u] = bf16_to_f32(x[static_cast<int64_t>(t + u) * d + i]);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float* g = dg + static_cast<int64_t>(t + u) * E + e0;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (e0 + q < E) acc[q] = fmaf(xv[u], g[q], acc[q]);
    }
  }
  for (; t < t1; ++t) {
    const float xv = bf16_to_f32(x[static_cast<int64_t>(t) * d + i]);
    const float* g = dg + static_cast<int64_t>(t) * E + e0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (e0 + q < E) acc[q] = fmaf(xv, g[q], acc[q]);
  }
  float* out = part + static_cast<int64_t>(blockIdx.z) * d * E;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    if (e0 + q < E) out[static_cast<int64_t>(i) * E + e0 + q] = acc[q];
}

__global__ __launch_bounds__(256) void dwgate_sum_kernel(const float* __restrict__ part,
                                                         float* __restrict__ dwg, int64_t n,
                                                         int S) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  float s = 0.f;
  int q = 0;
  for (; q + 8 <= S; q += 8) {
    float v[8];                                  // the loads first, the adds in order
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(q + u) * n + idx];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; q < S; ++q) s += part[q * n + idx];
  dwg[idx] = s;
}

// Token slices of dwgate_kernel: about 2048 blocks in all, at least 64
// tokens a slice.
int dwgate_slices(int64_t T, int64_t d, int E) {
  const int64_t blocks0 = ((d + 255) / 256) * ((E + 7) / 8);
  const int64_t s = std::min<int64_t>((T + 63) / 64, (2048 + blocks0 - 1) / blocks0);
  return static_cast<int>(std::max<int64_t>(1, s));
}

size_t align256b(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

}  // namespace

hipError_t launch_combine_backward(int64_t T, int64_t d, int E_shared, int k, const void* dy,
                                   const void* y_perm, const int32_t* row_of_pair,
                                   const float* topk_w, void* dy_perm, float* dtopk_w,
                                   hipStream_t s) {
  hipLaunchKernelGGL(combine_bwd_kernel, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(256), 0,
                     s, static_cast<const u32x4_t*>(dy), static_cast<const u32x4_t*>(y_perm),
                     row_of_pair, topk_w, static_cast<u32x4_t*>(dy_perm), dtopk_w,
                     static_cast<int>(T), k, E_shared, static_cast<int>(d / 8));
  return hipGetLastError();
}

hipError_t launch_route_backward(int64_t T, int64_t d, int E, int E_shared, int k, const void* x,
                                 const void* w_gate, const float* logits,
                                 const int32_t* topk_idx, const float* topk_w,
                                 const float* dtopk_w, const int32_t* counts,
                                 const int32_t* row_of_pair, const void* dx_perm,
                                 const void* dx_shared, float alpha, float beta, void* dx,
                                 float* dw_gate, void* ws, hipStream_t s) {
  float* dg = static_cast<float*>(ws);
  const unsigned tb = static_cast<unsigned>((T + 3) / 4);
  hipLaunchKernelGGL(route_dg_kernel, dim3(tb), dim3(256), 0, s, logits, topk_idx, topk_w,
                     dtopk_w, counts, dg, static_cast<int>(T), E, k, alpha, beta);
  hipLaunchKernelGGL(dx_kernel, dim3(tb), dim3(256), 0, s, static_cast<const u32x4_t*>(dx_perm),
                     static_cast<const u32x4_t*>(dx_shared), row_of_pair, dg,
                     static_cast<const uint16_t*>(w_gate), static_cast<u32x4_t*>(dx),
                     static_cast<int>(T), E, k, E_shared, static_cast<int>(d / 8));
  const int S = dwgate_slices(T, d, E);
  const int chunk = static_cast<int>((T + S - 1) / S);
  float* part = S > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                 align256b(static_cast<size_t>(T) * E * 4))
                      : dw_gate;
  hipLaunchKernelGGL(dwgate_kernel,
                     dim3(static_cast<unsigned>((d + 255) / 256), static_cast<unsigned>((E + 7) / 8),
                          static_cast<unsigned>(S)),
                     dim3(256), 0, s, static_cast<const uint16_t*>(x), dg, part,
                     static_cast<int>(T), static_cast<int>(d), E, chunk);
  if (S > 1) {
    const int64_t n = d * E;
    hipLaunchKernelGGL(dwgate_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                       0, s, part, dw_gate, n, S);
  }
  return hipGetLastError();
}

size_t route_backward_workspace_bytes(int64_t T, int64_t d, int E) {
  const int S = dwgate_slices(T, d, E);
  const size_t dg = align256b(static_cast<size_t>(T) * E * sizeof(float));
  return dg + (S > 1 ? static_cast<size_t>(S) * d * E * sizeof(float) : 0);
}

}  // namespace moe
