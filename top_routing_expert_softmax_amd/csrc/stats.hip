// Load-balance statistics and router z-loss, "MoE routing math" sections
// 3.2 (f_i, P_i, L_balance) and 4.3 (drop rate), "MoE deep dive" section 3.2
// (z-loss), all unscaled.
//
// Pass 1: each block takes a contiguous token range; one wavefront per
// token computes softmax and log-sum-exp in fp32 (each lane holds up to four
// logits), and fp64 per-lane accumulators collect sum_t p_ti and sum_t lse^2.
// The block folds its four waves in a fixed order into one partial row.
// Pass 2: one block adds the partial rows and forms f, P, L_balance, z and
// the drop rate in fp64, always in the same order (the result is
// deterministic).
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWavesS = 4;

__global__ __launch_bounds__(kWavesS * kWave) void stats_partial_kernel(
    const float* __restrict__ logits, double* __restrict__ part_P,
    double* __restrict__ part_z, int nT, int E, int tokens_per_block) {
  __shared__ double sP[kWavesS][256];
  __shared__ double sz[kWavesS];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  double accP[4] = {0.0, 0.0, 0.0, 0.0};
  double accz = 0.0;
  const int tb0 = blockIdx.x * tokens_per_block;
  const int tb1 = min(nT, tb0 + tokens_per_block);
  for (int t = tb0 + wave; t < tb1; t += kWavesS) {
    const float* row = logits + static_cast<int64_t>(t) * E;
    float g[4];
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane + kWave * r;
      g[r] = (e < E) ? row[e] : -INFINITY;
      m = fmaxf(m, g[r]);
    }
    m = wave_max(m);
    float ex[4];
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane + kWave * r;
      ex[r] = (e < E) ? expf(g[r] - m) : 0.f;
      s += ex[r];
    }
    s = wave_sum(s);
    const float inv = 1.0f / s;
#pragma unroll
    for (int r = 0; r < 4; ++r) accP[r] += static_cast<double>(ex[r] * inv);
    const double lse = static_cast<double>(m) + log(static_cast<double>(s));
    accz += lse * lse;   // same value on every lane; lane 0's copy is used
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane + kWave * r;
    if (e < E) sP[wave][e] = accP[r];
  }
  if (lane == 0) sz[wave] = accz;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double v = 0.0;
    for (int w = 0; w < kWavesS; ++w) v += sP[w][e];
    part_P[static_cast<int64_t>(blockIdx.x) * E + e] = v;
  }
  if (threadIdx.x == 0) {
    double v = 0.0;
    for (int w = 0; w < kWavesS; ++w) v += sz[w];
    part_z[blockIdx.x] = v;
  }
}

// 1024 threads: thread (j, e) with j = tid / 256 sums partial rows
// b = j, j+4, j+8, ... of expert e into eight fixed accumulators; the four
// j-sums and the accumulators are combined in a fixed order.
__global__ __launch_bounds__(1024) void stats_final_kernel(
    const double* __restrict__ part_P, const double* __restrict__ part_z,
    const int32_t* __restrict__ counts, float* __restrict__ f, float* __restrict__ P,
    double* __restrict__ scalars, int nblk, int nT, int E, int k, int cap) {
  __shared__ double sj[4][256];
  __shared__ double zj[4];
  __shared__ double fp[256];
  __shared__ double dr[256];
  const int e = threadIdx.x & 255;
  const int j = threadIdx.x >> 8;
  {
    double acc8[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    double z8[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int b0 = j; b0 < nblk; b0 += 32) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int b = b0 + 4 * q;
        if (b < nblk) {
          if (e < E) acc8[q] += part_P[static_cast<int64_t>(b) * E + e];
          if (e == 0) z8[q] += part_z[b];
        }
      }
    }
    sj[j][e] = ((acc8[0] + acc8[1]) + (acc8[2] + acc8[3])) + ((acc8[4] + acc8[5]) + (acc8[6] + acc8[7]));
    if (e == 0) zj[j] = ((z8[0] + z8[1]) + (z8[2] + z8[3])) + ((z8[4] + z8[5]) + (z8[6] + z8[7]));
  }
  __syncthreads();
  if (j == 0) {
    double fP = 0.0, drop = 0.0;
    if (e < E) {
      const double sumP = (sj[0][e] + sj[1][e]) + (sj[2][e] + sj[3][e]);
      const double Pe = sumP / nT;
      const double fe = static_cast<double>(counts[e]) / nT;
      f[e] = static_cast<float>(fe);
      P[e] = static_cast<float>(Pe);
      fP = fe * Pe;
      drop = static_cast<double>(max(0, counts[e] - cap));
    }
    fp[e] = fP;
    dr[e] = drop;
  }
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) {
      fp[threadIdx.x] += fp[threadIdx.x + off];
      dr[threadIdx.x] += dr[threadIdx.x + off];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double z = (zj[0] + zj[1]) + (zj[2] + zj[3]);
    scalars[0] = static_cast<double>(E) * fp[0];
    scalars[1] = z / nT;
    scalars[2] = dr[0] / (static_cast<double>(nT) * k);
  }
}

int stats_blocks(int64_t T, int* tokens_per_block) {
  int64_t tpb = kWavesS;
  while ((T + tpb - 1) / tpb > kStatsBlocks) tpb += kWavesS;
  *tokens_per_block = static_cast<int>(tpb);
  return static_cast<int>((T + tpb - 1) / tpb);
}

}  // namespace

size_t stats_workspace_bytes(int64_t /*T*/, int E) {
  return static_cast<size_t>(kStatsBlocks) * (E + 1) * sizeof(double);
}

hipError_t launch_aux_stats(int64_t T, int E, int k, int64_t cap, const float* logits,
                            const int32_t* counts, float* f, float* P, double* scalars,
                            void* ws, hipStream_t s) {
  int tpb = 0;
  const int nblk = stats_blocks(T, &tpb);
  double* part_P = static_cast<double*>(ws);
  double* part_z = part_P + static_cast<size_t>(kStatsBlocks) * E;
  hipLaunchKernelGGL(stats_partial_kernel, dim3(nblk), dim3(kWavesS * kWave), 0, s, logits,
                     part_P, part_z, static_cast<int>(T), E, tpb);
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(1024), 0, s, part_P, part_z, counts, f,
                     P, scalars, nblk, static_cast<int>(T), E, k, static_cast<int>(cap));
  return hipGetLastError();
}

}  // namespace moe
