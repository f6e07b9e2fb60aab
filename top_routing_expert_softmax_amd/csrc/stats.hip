// Load-balance statistics and router z-loss, "MoE routing math" sections
// 3.2 (f_i, P_i, L_balance) and 4.3 (drop rate), "MoE deep dive" section 3.2
// (z-loss), all unscaled.
//
// Pass 1: each block takes a contiguous token range; a wavefront computes
// softmax and log-sum-exp in fp32 for one token (each lane holding up to
// four logits) or, when E <= 64, for four tokens at once (one per logit
// slot), and fp64 per-lane accumulators collect sum_t p_ti and
// sum_t lse^2.
// The block folds its four waves in a fixed order into one partial row.
// Pass 2: one block adds the partial rows (spread over all its threads
// whatever E is) and forms f, P, L_balance, z and the drop rate in fp64,
// always in the same order (the result is deterministic).
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWavesS = 4;

// Softmax and log-sum-exp of the tokens a lane's four logit slots hold:
// with E <= 64 slot r is token t + r (expert lane), otherwise the four
// slots are experts lane + 64 r of token t.  The wave reductions are DPP
// ones (fixed order); the four tokens' reductions run side by side.
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
  if (E <= kWave) {
    for (int t = tb0 + 4 * wave; t < tb1; t += 4 * kWavesS) {
      float g[4], m[4], ex[4], s[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        g[r] = lane < E && t + r < tb1 ? logits[static_cast<int64_t>(t + r) * E + lane] : -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) m[r] = wave_max_dpp(g[r]);
#pragma unroll
      for (int r = 0; r < 4; ++r) ex[r] = lane < E && t + r < tb1 ? expf(g[r] - m[r]) : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = wave_sum_dpp(ex[r]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (t + r < tb1) {
          accP[0] += static_cast<double>(ex[r] * (1.0f / s[r]));
          const double lse = static_cast<double>(m[r]) + log(static_cast<double>(s[r]));
          accz += lse * lse;   // same value on every lane; lane 0's copy is used
        }
      }
    }
  } else {
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
      m = wave_max_dpp(m);
      float ex[4];
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = lane + kWave * r;
        ex[r] = (e < E) ? expf(g[r] - m) : 0.f;
        s += ex[r];
      }
      s = wave_sum_dpp(s);
      const float inv = 1.0f / s;
#pragma unroll
      for (int r = 0; r < 4; ++r) accP[r] += static_cast<double>(ex[r] * inv);
      const double lse = static_cast<double>(m) + log(static_cast<double>(s));
      accz += lse * lse;
    }
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

// 1024 threads: with EP = E rounded up to a power of two (at most 256) and
// G = 1024 / EP groups, thread (g, e) = (tid / EP, tid % EP) sums the
// partial rows b = g, g + G, g + 2G, ... of expert e into eight fixed
// accumulators (its loads all issued before the adds), and the G group
// sums are folded in a fixed tree, so the result does not depend on
// scheduling.
__global__ __launch_bounds__(1024) void stats_final_kernel(
    const double* __restrict__ part_P, const double* __restrict__ part_z,
    const int32_t* __restrict__ counts, float* __restrict__ f, float* __restrict__ P,
    double* __restrict__ scalars, int nblk, int nT, int E, int k, int cap, int EP) {
  __shared__ double sj[1024];
  __shared__ double zj[1024];
  __shared__ double fp[256];
  __shared__ double dr[256];
  const int G = 1024 / EP;
  const int e = threadIdx.x % EP;
  const int g = threadIdx.x / EP;
  {
    double acc8[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    double z8[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    // every load in bounds and unconditional, so the eight are in flight
    // together; rows past nblk and experts past E add nothing
    const int ec = min(e, E - 1);
    for (int b0 = g; b0 < nblk; b0 += 8 * G) {
      double vP[8], vz[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int b = min(b0 + q * G, nblk - 1);
        vP[q] = part_P[static_cast<int64_t>(b) * E + ec];
        vz[q] = part_z[b];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (b0 + q * G < nblk) {
          if (e < E) acc8[q] += vP[q];
          if (e == 0) z8[q] += vz[q];
        }
      }
    }
    sj[threadIdx.x] = ((acc8[0] + acc8[1]) + (acc8[2] + acc8[3])) +
                      ((acc8[4] + acc8[5]) + (acc8[6] + acc8[7]));
    zj[threadIdx.x] = ((z8[0] + z8[1]) + (z8[2] + z8[3])) + ((z8[4] + z8[5]) + (z8[6] + z8[7]));
  }
  __syncthreads();
  // fold the groups: element (g, e) += (g + h, e) for h = G/2, G/4, ..., 1
  for (int h = G / 2; h > 0; h >>= 1) {
    if (g < h) {
      sj[threadIdx.x] += sj[threadIdx.x + h * EP];
      zj[threadIdx.x] += zj[threadIdx.x + h * EP];
    }
    __syncthreads();
  }
  if (threadIdx.x < 256) {
    double fP = 0.0, drop = 0.0;
    const int ee = threadIdx.x;
    if (ee < E) {
      const double Pe = sj[ee] / nT;
      const double fe = static_cast<double>(counts[ee]) / nT;
      f[ee] = static_cast<float>(fe);
      P[ee] = static_cast<float>(Pe);
      fP = fe * Pe;
      drop = static_cast<double>(max(0, counts[ee] - cap));
    }
    fp[ee] = fP;
    dr[ee] = drop;
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
    scalars[0] = static_cast<double>(E) * fp[0];
    scalars[1] = zj[0] / nT;
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
  int EP = 1;
  while (EP < E) EP <<= 1;
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(1024), 0, s, part_P, part_z, counts, f,
                     P, scalars, nblk, static_cast<int>(T), E, k, static_cast<int>(cap), EP);
  return hipGetLastError();
}

}  // namespace moe
