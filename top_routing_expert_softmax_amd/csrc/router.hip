// Fused router: logits g = x W_gate, then top-k and renormalised weights.
// "MoE routing math", section 2.1.
//
// One block owns kTW tokens and all E experts.  Its waves split d into
// contiguous ranges; inside a wave, lane = es + ES * ds, where es picks EPL
// consecutive experts and ds interleaves 8-element chunks of d.  Each lane
// keeps kTW x EPL fp32 accumulators and uses plain fp32 FMAs (no MFMA), so
// on the dyadic input grid every partial sum is exact and the logits do not
// depend on the summation order.  Partials are reduced across ds lanes with
// shuffles, across waves through LDS, and the block then writes the logits.
// The epilogue gives each token one wavefront: every lane holds up to four
// logits, k rounds of a wave-wide max over (logit, -index) keys select the
// experts (larger logit first, ties to the lower index), and the weights are
// exp(g_j - g_max) / sum over the selected j.
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTW = 8;          // tokens per block
constexpr int kMaxWavesR = 8;   // waves per block at most

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16lo(q.x); v[1] = bf16hi(q.x);
  v[2] = bf16lo(q.y); v[3] = bf16hi(q.y);
  v[4] = bf16lo(q.z); v[5] = bf16hi(q.z);
  v[6] = bf16lo(q.w); v[7] = bf16hi(q.w);
}

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load1(const float* p) { return *p; }

// Eight consecutive x values of one token: bf16 kept packed (4 registers),
// fp32 as 8 registers.
template <typename T>
struct XChunk;

template <>
struct XChunk<uint16_t> {
  u32x4_t q;
  __device__ __forceinline__ void load(const uint16_t* p) { q = *reinterpret_cast<const u32x4_t*>(p); }
  __device__ __forceinline__ void zero() { q = u32x4_t{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ float get(int u) const {
    const uint32_t w = q[u >> 1];
    return (u & 1) ? bf16hi(w) : bf16lo(w);
  }
};

template <>
struct XChunk<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const f32x4_t*>(p)[0];
    b = reinterpret_cast<const f32x4_t*>(p)[1];
  }
  __device__ __forceinline__ void zero() { a = f32x4_t{0.f, 0.f, 0.f, 0.f}; b = a; }
  __device__ __forceinline__ float get(int u) const { return u < 4 ? a[u] : b[u - 4]; }
};

// EPL consecutive experts of one W_gate row; vec: row is 16-byte aligned
// and all EPL experts exist.
template <int EPL>
__device__ __forceinline__ void load_w(const uint16_t* row, int e0, int E, bool vec,
                                       float (&w)[EPL]) {
  if constexpr (EPL == 8) {
    if (vec) { load8(row + e0, w); return; }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) w[e] = (e0 + e < E) ? load1(row + e0 + e) : 0.f;
}

template <int EPL>
__device__ __forceinline__ void load_w(const float* row, int e0, int E, bool vec,
                                       float (&w)[EPL]) {
  if constexpr (EPL == 8) {
    if (vec) { load8(row + e0, w); return; }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) w[e] = (e0 + e < E) ? load1(row + e0 + e) : 0.f;
}

template <typename T, int EPL>
__global__ __launch_bounds__(kMaxWavesR * kWave) void router_kernel(
    const T* __restrict__ x, const T* __restrict__ wg, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int nT, int d,
    int E, int k, int ES, int chunks_per_wave) {
  extern __shared__ float smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  const int DS = kWave / ES;
  const int es = lane % ES;
  const int ds = lane / ES;
  const int E_pad = ES * EPL;
  const int e0 = es * EPL;
  const int t0 = blockIdx.x * kTW;
  const bool vec_w = (E % 8 == 0);

  float acc[kTW][EPL];
#pragma unroll
  for (int t = 0; t < kTW; ++t)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[t][e] = 0.f;

  const int nchunk = d / 8;
  const int c_begin = wave * chunks_per_wave;
  const int c_end = min(nchunk, c_begin + chunks_per_wave);
  if (e0 < E) {
    for (int c = c_begin + ds; c < c_end; c += DS) {
      const int i0 = c * 8;
      XChunk<T> xv[kTW];
#pragma unroll
      for (int t = 0; t < kTW; ++t) {
        if (t0 + t < nT) xv[t].load(x + static_cast<int64_t>(t0 + t) * d + i0);
        else xv[t].zero();
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float w[EPL];
        load_w<EPL>(wg + static_cast<int64_t>(i0 + u) * E, e0, E, vec_w, w);
#pragma unroll
        for (int t = 0; t < kTW; ++t) {
          const float xu = xv[t].get(u);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[t][e] = fmaf(xu, w[e], acc[t][e]);
        }
      }
    }
  }
  // Sum over the ds lanes that share es (lane bits above log2(ES)).
  for (int off = ES; off < kWave; off <<= 1) {
#pragma unroll
    for (int t = 0; t < kTW; ++t)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[t][e] += __shfl_xor(acc[t][e], off, kWave);
  }
  float* red = smem;                              // [nwaves][kTW][E_pad]
  float* lg = smem + nwaves * kTW * E_pad;        // [kTW][E_pad]
  if (ds == 0) {
#pragma unroll
    for (int t = 0; t < kTW; ++t)
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[(wave * kTW + t) * E_pad + e0 + e] = acc[t][e];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < kTW * E_pad; q += blockDim.x) {
    float s = 0.f;
    for (int w = 0; w < nwaves; ++w) s += red[w * kTW * E_pad + q];
    lg[q] = s;
    const int t = q / E_pad, e = q % E_pad;
    if (t0 + t < nT && e < E) logits[static_cast<int64_t>(t0 + t) * E + e] = s;
  }
  __syncthreads();

  // Top-k and renormalisation, one wavefront per token.
  for (int tt = wave; tt < kTW; tt += nwaves) {
    const int t = t0 + tt;
    if (t >= nT) break;
    const float* row = lg + tt * E_pad;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane + kWave * r;
      v[r] = (e < E) ? row[e] : 0.f;
    }
    uint32_t taken = 0;
    float gmax = 0.f, wsum = 0.f, my_w = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = lane + kWave * r;
        if (e < E && !((taken >> r) & 1u)) {
          const uint64_t key = (static_cast<uint64_t>(f32_order_key(v[r])) << 32) |
                               static_cast<uint64_t>(0xFFFFFFFFu - static_cast<uint32_t>(e));
          best = key > best ? key : best;
        }
      }
      best = wave_max_u64(best);
      const int e_sel = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
      const float g_sel = row[e_sel];
      if ((e_sel & (kWave - 1)) == lane) taken |= 1u << (e_sel / kWave);
      if (j == 0) gmax = g_sel;
      const float ex = expf(g_sel - gmax);
      wsum += ex;
      if (lane == j) { my_w = ex; my_e = e_sel; }
    }
    if (lane < k) {
      topk_idx[static_cast<int64_t>(t) * k + lane] = my_e;
      topk_w[static_cast<int64_t>(t) * k + lane] = my_w / wsum;
    }
  }
}

template <typename T, int EPL>
hipError_t launch_t(int64_t T_, int64_t d, int E, int k, const void* x, const void* wg,
                    float* logits, int32_t* idx, float* w, int ES, hipStream_t s) {
  const int E_pad = ES * EPL;
  const int DS = kWave / ES;
  const int nblocks = static_cast<int>((T_ + kTW - 1) / kTW);
  const int nchunk = static_cast<int>(d / 8);
  // Enough waves to fill the chip, no more than the chunks can feed, and
  // the reduction buffers within 64 KB of LDS.
  int nwaves = (2048 + nblocks - 1) / nblocks;
  nwaves = min(nwaves, kMaxWavesR);
  nwaves = min(nwaves, max(1, nchunk / DS));
  const int lds_per_wave = kTW * E_pad * 4;
  nwaves = min(nwaves, 65536 / lds_per_wave - 1);
  nwaves = max(nwaves, 1);
  int cpw = (nchunk + nwaves - 1) / nwaves;
  cpw = ((cpw + DS - 1) / DS) * DS;
  const size_t lds = static_cast<size_t>(nwaves + 1) * lds_per_wave;
  hipLaunchKernelGGL((router_kernel<T, EPL>), dim3(nblocks), dim3(nwaves * kWave), lds, s,
                     static_cast<const T*>(x), static_cast<const T*>(wg), logits, idx, w,
                     static_cast<int>(T_), static_cast<int>(d), E, k, ES, cpw);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_epl(int64_t T_, int64_t d, int E, int k, const void* x, const void* wg,
                        float* logits, int32_t* idx, float* w, hipStream_t s) {
  int E_pad = 1;
  while (E_pad < E) E_pad <<= 1;
  if (E_pad >= 8) return launch_t<T, 8>(T_, d, E, k, x, wg, logits, idx, w, E_pad / 8, s);
  if (E_pad == 4) return launch_t<T, 4>(T_, d, E, k, x, wg, logits, idx, w, 1, s);
  if (E_pad == 2) return launch_t<T, 2>(T_, d, E, k, x, wg, logits, idx, w, 1, s);
  return launch_t<T, 1>(T_, d, E, k, x, wg, logits, idx, w, 1, s);
}

}  // namespace

hipError_t launch_route(int64_t T, int64_t d, int E, int k, bool bf16, const void* x,
                        const void* w_gate, float* logits, int32_t* topk_idx,
                        float* topk_w, hipStream_t s) {
  if (bf16)
    return dispatch_epl<uint16_t>(T, d, E, k, x, w_gate, logits, topk_idx, topk_w, s);
  return dispatch_epl<float>(T, d, E, k, x, w_gate, logits, topk_idx, topk_w, s);
}

}  // namespace moe
