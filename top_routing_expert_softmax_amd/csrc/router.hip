// Fused router: logits g = x W_gate, then top-k and renormalised weights.
// "MoE routing math", section 2.1.
//
// A block owns kTW tokens and all E experts over a range of d.  Its waves
// split that range; inside a wave, lane = es + ES * ds, where es picks EPL
// consecutive experts and ds interleaves 8-element chunks of d.  Each lane
// keeps kTW x EPL fp32 accumulators and uses plain fp32 FMAs (no MFMA), so
// on the dyadic input grid every partial sum is exact and the logits do not
// depend on the summation order.  Partials are reduced across ds lanes with
// shuffles and across waves through LDS.
//
// Many tokens (prefill): one block per kTW tokens covers all of d and runs
// the top-k epilogue itself.  Few tokens (decode): d is also split across S
// blocks that write partial logits to the workspace; a select kernel adds
// the S partials in a fixed order and runs the same top-k.
//
// Top-k: one wavefront per token, each lane holding up to four logits; k
// rounds of a wave-wide max over (order key of the logit, -index) pick the
// experts, larger logit first and ties to the lower index; the weights are
// exp(g_j - g_max) / sum over the selected j.
//
// DeepSeek-V3 gate ("CMU 11-868 Lecture 17", section 5.3; the bias of
// section 3.4), same logits: affinity s = sigmoid(g) (evaluated in fp64,
// rounded once to fp32), biased = s + b in fp32; a group's score is the
// fp32 sum of its two largest biased scores; topk_groups groups are kept
// (ties to the lower group); the k largest biased scores inside them are
// chosen (ties to the lower expert); the weights are the chosen unbiased
// affinities over their sum, times route_scale.
#include <math.h>

#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTW = 8;          // tokens per block
constexpr int kMaxWavesR = 8;   // waves per block at most
constexpr int kMaxSplits = 64;  // d-splits at most (decode)
constexpr int kRouterSplitBlocks = 256;   // blocks the d-split aims for

}  // namespace

// Which top-k follows the logits (see the file comment).
struct GateParams {
  int v3;                 // 0: softmax top-k; 1: DeepSeek-V3 gate; 2: logits only
  const float* bias;      // [E] selection bias (V3)
  int n_groups, topk_groups;
  float route_scale;
};

namespace {

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const u32x4_t q = *reinterpret_cast<const u32x4_t*>(p);
  v[0] = bf16lo(q[0]); v[1] = bf16hi(q[0]);
  v[2] = bf16lo(q[1]); v[3] = bf16hi(q[1]);
  v[4] = bf16lo(q[2]); v[5] = bf16hi(q[2]);
  v[6] = bf16lo(q[3]); v[7] = bf16hi(q[3]);
}

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0];
  const f32x4_t b = reinterpret_cast<const f32x4_t*>(p)[1];
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
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

// EPL consecutive experts of one W_gate row; vec: the row is 16-byte
// aligned and all EPL experts exist.
template <int EPL, typename T>
__device__ __forceinline__ void load_w(const T* row, int e0, int E, bool vec, float (&w)[EPL]) {
  if constexpr (EPL == 8) {
    if (vec) { load8(row + e0, w); return; }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) w[e] = (e0 + e < E) ? load1(row + e0 + e) : 0.f;
}

// One reduce-scatter round per call over the lane bit `off` (then the next
// one, with half the values): the lane with the bit set keeps the upper H
// of its 2H values, the other the lower H, and each adds its partner's copy
// of the half it keeps.  base: index of v[0] among the original values.
// Stops early once off reaches the wave width.
template <int H>
__device__ __forceinline__ void scatter_rounds(float* v, int lane, int& off, int& base) {
  if constexpr (H >= 1) {
    if (off >= kWave) return;
    const bool hi = (lane & off) != 0;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const float send = hi ? v[j] : v[j + H];
      const float keep = hi ? v[j + H] : v[j];
      v[j] = keep + __shfl_xor(send, off, kWave);
    }
    if (hi) base += H;
    off <<= 1;
    scatter_rounds<H / 2>(v, lane, off, base);
  }
}

__device__ __forceinline__ float from_order_key(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

// Top-k of one token held by one wavefront: lane holds logits of experts
// lane + 64 r (r < 4) in v[r].  Writes k ids and renormalised weights.
__device__ __forceinline__ void topk_select(const float (&v)[4], int E, int k, int lane,
                                            int32_t* __restrict__ idx_row,
                                            float* __restrict__ w_row) {
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
    const float g_sel = from_order_key(static_cast<uint32_t>(best >> 32));
    if ((e_sel & (kWave - 1)) == lane) taken |= 1u << (e_sel / kWave);
    if (j == 0) gmax = g_sel;
    const float ex = expf(g_sel - gmax);
    wsum += ex;
    if (lane == j) { my_w = ex; my_e = e_sel; }
  }
  if (lane < k) {
    idx_row[lane] = my_e;
    w_row[lane] = my_w / wsum;
  }
}

// DeepSeek-V3 gate of one token held by one wavefront: g_row (LDS) holds
// the E logits, scratch (LDS, E floats) is this wave's own.
__device__ __forceinline__ void v3_select(const float* g_row, float* scratch, const GateParams& gp,
                                          int E, int k, int lane, int32_t* __restrict__ idx_row,
                                          float* __restrict__ w_row) {
  float s[4], bsc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane + kWave * r;
    s[r] = 0.f;
    bsc[r] = 0.f;
    if (e < E) {
      s[r] = static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(g_row[e]))));
      bsc[r] = s[r] + gp.bias[e];
      scratch[e] = bsc[r];
    }
  }
  // the scratch row is read by other lanes of this wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int G = E / gp.n_groups;
  // lane q < n_groups: the two largest biased scores of group q
  uint32_t gkey = 0;
  if (lane < gp.n_groups) {
    float t1 = -INFINITY, t2 = -INFINITY;
    for (int i = 0; i < G; ++i) {
      const float v = scratch[lane * G + i];
      if (v > t1) { t2 = t1; t1 = v; }
      else if (v > t2) { t2 = v; }
    }
    gkey = f32_order_key(t1 + t2);
  }
  // keep topk_groups groups: rounds of a wave max over (score, -group)
  uint64_t kept = 0;
  for (int j = 0; j < gp.topk_groups; ++j) {
    uint64_t key = 0;
    if (lane < gp.n_groups && !((kept >> lane) & 1ull))
      key = (static_cast<uint64_t>(gkey) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - lane);
    key = wave_max_u64(key);
    kept |= 1ull << (0xFFFFFFFFu - static_cast<uint32_t>(key));
  }
  // k experts of the kept groups by biased score
  uint32_t taken = 0;
  float wsum = 0.f, my_s = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
    float best_s = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane + kWave * r;
      if (e < E && ((kept >> (e / G)) & 1ull) && !((taken >> r) & 1u)) {
        const uint64_t key = (static_cast<uint64_t>(f32_order_key(bsc[r])) << 32) |
                             static_cast<uint64_t>(0xFFFFFFFFu - static_cast<uint32_t>(e));
        if (key > best) { best = key; best_s = s[r]; }
      }
    }
    const uint64_t wbest = wave_max_u64(best);
    const int e_sel = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(wbest));
    // the lane that holds the winner broadcasts its affinity
    const int owner = e_sel & (kWave - 1);
    const float s_sel = __shfl(best_s, owner, kWave);
    if (owner == lane) taken |= 1u << (e_sel / kWave);
    wsum += s_sel;
    if (lane == j) { my_s = s_sel; my_e = e_sel; }
  }
  if (lane < k) {
    idx_row[lane] = my_e;
    w_row[lane] = my_s / wsum * gp.route_scale;
  }
}

// SPLIT = false: all of d, then the top-k epilogue.  SPLIT = true: the
// chunk range [blockIdx.y * cps, +cps) of d, partial logits to
// partial[blockIdx.y][t][e].
template <typename T, int EPL, bool SPLIT>
__global__ __launch_bounds__(kMaxWavesR * kWave) void router_kernel(
    const T* __restrict__ x, const T* __restrict__ wg, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, float* __restrict__ partial,
    int nT, int d, int E, int k, int ES, int chunks_per_wave, int chunks_per_split,
    GateParams gp) {
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
  const int split_begin = SPLIT ? blockIdx.y * chunks_per_split : 0;
  const int split_end = SPLIT ? min(nchunk, split_begin + chunks_per_split) : nchunk;
  const int c_begin = split_begin + wave * chunks_per_wave;
  const int c_end = min(split_end, c_begin + chunks_per_wave);
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
  // Sum over the ds lanes that share es (lane bits above log2(ES)) by
  // reduce-scatter: each round hands half of the lane's remaining sums to
  // its partner and adds the partner's copy of the other half, so the
  // lanes end up holding distinct, fully summed (token, expert) values.
  constexpr int V = kTW * EPL;
  float v[V];
#pragma unroll
  for (int t = 0; t < kTW; ++t)
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[t * EPL + e] = acc[t][e];
  int off = ES, base = 0;
  scatter_rounds<V / 2>(v, lane, off, base);
  int rounds = 0;                                 // rounds that halved
  while ((ES << rounds) < off) ++rounds;
  const int R = V >> rounds;                      // sums this lane holds
  // more ds lanes than values: the remaining rounds add whole sums
  for (; off < kWave; off <<= 1) v[0] += __shfl_xor(v[0], off, kWave);
  float* red = smem;                              // [nwaves][kTW][E_pad]
  float* lg = smem + nwaves * kTW * E_pad;        // [kTW][E_pad]
  if ((ds >> rounds) == 0) {                      // one writer per value
#pragma unroll
    for (int j = 0; j < V; ++j) {
      if (j < R) {
        const int q = base + j, t = q / EPL, e = q % EPL;
        red[(wave * kTW + t) * E_pad + e0 + e] = v[j];
      }
    }
  }
  __syncthreads();
  float* dst = SPLIT ? partial + static_cast<int64_t>(blockIdx.y) * nT * E : logits;
  for (int q = threadIdx.x; q < kTW * E_pad; q += blockDim.x) {
    float s = 0.f;
    for (int w = 0; w < nwaves; ++w) s += red[w * kTW * E_pad + q];
    lg[q] = s;
    const int t = q / E_pad, e = q % E_pad;
    if (t0 + t < nT && e < E) dst[static_cast<int64_t>(t0 + t) * E + e] = s;
  }
  if (SPLIT || gp.v3 == 2) return;
  __syncthreads();
  for (int tt = wave; tt < kTW; tt += nwaves) {
    const int t = t0 + tt;
    if (t >= nT) break;
    const float* row = lg + tt * E_pad;
    if (gp.v3 == 1) {
      // the per-wave reduction rows are free by now: scratch for the gate
      v3_select(row, red + wave * kTW * E_pad, gp, E, k, lane,
                topk_idx + static_cast<int64_t>(t) * k, topk_w + static_cast<int64_t>(t) * k);
      continue;
    }
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane + kWave * r;
      v[r] = (e < E) ? row[e] : 0.f;
    }
    topk_select(v, E, k, lane, topk_idx + static_cast<int64_t>(t) * k,
                topk_w + static_cast<int64_t>(t) * k);
  }
}

// Decode: logits = sum over the S d-splits, then top-k.  One block of 256
// threads per token, thread e < E adds partial[s][t][e] into eight
// accumulators (s mod 8) that are combined in a fixed order; wavefront 0
// then selects from the LDS copy of the row.
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ partial, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int nT, int E, int k, int S,
    GateParams gp) {
  __shared__ float row[256];
  __shared__ float scratch[256];
  const int t = blockIdx.x;
  const int e = threadIdx.x;
  float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (e < E) {
    for (int s0 = 0; s0 < S; s0 += 8) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (s0 + q < S) s8[q] += partial[(static_cast<int64_t>(s0 + q) * nT + t) * E + e];
    }
  }
  const float g = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
  if (e < E) logits[static_cast<int64_t>(t) * E + e] = g;
  if (gp.v3 == 2) return;
  row[e] = g;
  __syncthreads();
  if (threadIdx.x < kWave && gp.v3 == 1) {
    v3_select(row, scratch, gp, E, k, threadIdx.x, topk_idx + static_cast<int64_t>(t) * k,
              topk_w + static_cast<int64_t>(t) * k);
  } else if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = row[lane + kWave * r];
    topk_select(v, E, k, lane, topk_idx + static_cast<int64_t>(t) * k,
                topk_w + static_cast<int64_t>(t) * k);
  }
}

struct RouterPlan {
  int E_pad, ES, EPL, DS;
  int nblocks, nchunk;
  int S, cps;               // d-splits and chunks per split
  int nwaves, cpw;
};

RouterPlan plan_router(int64_t T, int64_t d, int E) {
  RouterPlan p;
  p.E_pad = 1;
  while (p.E_pad < E) p.E_pad <<= 1;
  p.EPL = p.E_pad >= 8 ? 8 : p.E_pad;
  p.ES = p.E_pad / p.EPL;
  p.DS = kWave / p.ES;
  p.nblocks = static_cast<int>((T + kTW - 1) / kTW);
  p.nchunk = static_cast<int>(d / 8);
  // split d across blocks when there are too few token blocks to fill
  // the chip (each split keeps at least one chunk per ds lane)
  p.S = 1;
  if (p.nblocks < 128) {
    p.S = (kRouterSplitBlocks + p.nblocks - 1) / p.nblocks;
    p.S = std::min(p.S, kMaxSplits);
    p.S = std::min(p.S, std::max(1, p.nchunk / p.DS));
  }
  p.cps = (p.nchunk + p.S - 1) / p.S;
  p.S = (p.nchunk + p.cps - 1) / p.cps;
  // enough waves to fill the chip, no more than the chunks can feed, and
  // the reduction buffers within 64 KB of LDS
  int nw = (2048 + p.nblocks * p.S - 1) / (p.nblocks * p.S);
  nw = std::min(nw, kMaxWavesR);
  nw = std::min(nw, std::max(1, p.cps / p.DS));
  const int lds_per_wave = kTW * p.E_pad * 4;
  nw = std::min(nw, 65536 / lds_per_wave - 1);
  p.nwaves = std::max(nw, 1);
  p.cpw = (p.cps + p.nwaves - 1) / p.nwaves;
  p.cpw = ((p.cpw + p.DS - 1) / p.DS) * p.DS;
  return p;
}

template <typename T, int EPL>
hipError_t launch_t(const RouterPlan& p, int64_t T_, int64_t d, int E, int k, const void* x,
                    const void* wg, float* logits, int32_t* idx, float* w, float* partial,
                    const GateParams& gp, hipStream_t s) {
  const size_t lds = static_cast<size_t>(p.nwaves + 1) * kTW * p.E_pad * 4;
  if (p.S == 1) {
    hipLaunchKernelGGL((router_kernel<T, EPL, false>), dim3(p.nblocks), dim3(p.nwaves * kWave),
                       lds, s, static_cast<const T*>(x), static_cast<const T*>(wg), logits, idx,
                       w, nullptr, static_cast<int>(T_), static_cast<int>(d), E, k, p.ES, p.cpw,
                       p.cps, gp);
  } else {
    hipLaunchKernelGGL((router_kernel<T, EPL, true>), dim3(p.nblocks, p.S),
                       dim3(p.nwaves * kWave), lds, s, static_cast<const T*>(x),
                       static_cast<const T*>(wg), logits, idx, w, partial, static_cast<int>(T_),
                       static_cast<int>(d), E, k, p.ES, p.cpw, p.cps, gp);
    hipLaunchKernelGGL(router_select_kernel, dim3(static_cast<unsigned>(T_)), dim3(256), 0, s,
                       partial, logits, idx, w, static_cast<int>(T_), E, k, p.S, gp);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_epl(int64_t T_, int64_t d, int E, int k, const void* x, const void* wg,
                        float* logits, int32_t* idx, float* w, float* partial,
                        const GateParams& gp, hipStream_t s) {
  const RouterPlan p = plan_router(T_, d, E);
  switch (p.EPL) {
    case 8: return launch_t<T, 8>(p, T_, d, E, k, x, wg, logits, idx, w, partial, gp, s);
    case 4: return launch_t<T, 4>(p, T_, d, E, k, x, wg, logits, idx, w, partial, gp, s);
    case 2: return launch_t<T, 2>(p, T_, d, E, k, x, wg, logits, idx, w, partial, gp, s);
    default: return launch_t<T, 1>(p, T_, d, E, k, x, wg, logits, idx, w, partial, gp, s);
  }
}

// Balance-bias step ("CMU 11-868 Lecture 17", section 3.4): thread e
// compares counts[e] * E with T * k (the mean load, exactly).
__global__ __launch_bounds__(256) void update_bias_kernel(const int32_t* __restrict__ counts,
                                                          float* __restrict__ bias, int E,
                                                          int64_t Tk, float gamma) {
  const int e = threadIdx.x;
  if (e >= E) return;
  const int64_t load = static_cast<int64_t>(counts[e]) * E;
  if (load > Tk) bias[e] = bias[e] - gamma;
  else if (load < Tk) bias[e] = bias[e] + gamma;
}

}  // namespace

size_t route_workspace_bytes(int64_t T, int64_t d, int E) {
  const RouterPlan p = plan_router(T, d, E);
  return p.S == 1 ? 0 : static_cast<size_t>(p.S) * T * E * sizeof(float);
}

hipError_t launch_route(int64_t T, int64_t d, int E, int k, bool bf16, const void* x,
                        const void* w_gate, float* logits, int32_t* topk_idx, float* topk_w,
                        void* ws, const GateParams& gp, hipStream_t s) {
  float* partial = static_cast<float*>(ws);
  if (bf16)
    return dispatch_epl<uint16_t>(T, d, E, k, x, w_gate, logits, topk_idx, topk_w, partial, gp,
                                  s);
  return dispatch_epl<float>(T, d, E, k, x, w_gate, logits, topk_idx, topk_w, partial, gp, s);
}

hipError_t launch_route_softmax(int64_t T, int64_t d, int E, int k, bool bf16, const void* x,
                                const void* w_gate, float* logits, int32_t* topk_idx,
                                float* topk_w, void* ws, hipStream_t s) {
  const GateParams gp{0, nullptr, 1, 1, 1.0f};
  return launch_route(T, d, E, k, bf16, x, w_gate, logits, topk_idx, topk_w, ws, gp, s);
}

hipError_t launch_route_v3(int64_t T, int64_t d, int E, int k, int n_groups, int topk_groups,
                           float route_scale, bool bf16, const void* x, const void* w_gate,
                           const float* bias, float* logits, int32_t* topk_idx, float* topk_w,
                           void* ws, hipStream_t s) {
  const GateParams gp{1, bias, n_groups, topk_groups, route_scale};
  return launch_route(T, d, E, k, bf16, x, w_gate, logits, topk_idx, topk_w, ws, gp, s);
}

hipError_t launch_logits(int64_t T, int64_t d, int E, bool bf16, const void* x,
                         const void* w_gate, float* logits, void* ws, hipStream_t s) {
  const GateParams gp{2, nullptr, 1, 1, 1.0f};
  return launch_route(T, d, E, 1, bf16, x, w_gate, logits, nullptr, nullptr, ws, gp, s);
}

hipError_t launch_update_bias(int64_t T, int E, int k, float gamma, const int32_t* counts,
                              float* bias, hipStream_t s) {
  hipLaunchKernelGGL(update_bias_kernel, dim3(1), dim3(256), 0, s, counts, bias, E, T * k, gamma);
  return hipGetLastError();
}

}  // namespace moe
