// Expert-choice routing: "MoE deep dive: routing mechanisms and load
// balancing", section 2.2.  The logits are transposed so experts come
// first and each expert takes the cap tokens with the largest logits
// (larger first, ties to the lower token index).  A chosen pair is weighted
// by the router probability softmax(g_t)_e (the listing leaves the weight
// open); a token that no expert chose gets no routed output.
//
// Selection, one block of 1024 threads per expert:
//   1. radix select (four 8-bit digits of the fp32 order key, most
//      significant first) finds K*, the key of the cap-th largest logit,
//      and how many of the keys equal to K* are taken;
//   2. every thread owns a contiguous run of tokens; block scans place the
//      keys above K* and the first (lowest-token) keys equal to K* into LDS;
//   3. a bitonic sort on (key, -token) orders the cap picks, larger first
//      (keys in registers and wave shuffles for strides below 64 when the
//      padded count fits the block).
// Keys compare exactly (the logits are fp32), so the choice is exact.
//
// Dispatch: expert e owns rows e*cap .. e*cap+cap-1 of x_perm; row_of_te and
// w_te ([T, E], -1 / 0 where expert e did not choose token t) let
// moe_combine add the expert outputs back with k = E.
#include <math.h>

#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kEcThreads = 1024;
constexpr int kEcWaves = kEcThreads / kWave;

// Exclusive scan over the 1024 threads of the block (tmp: kEcWaves + 1 ints
// of LDS); *total receives the block sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int n = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += n;
  }
  if (lane == kWave - 1) tmp[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kEcWaves ? tmp[lane] : 0;
    int wi = w;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int n = __shfl_up(wi, off, kWave);
      if (lane >= off) wi += n;
    }
    if (lane < kEcWaves) tmp[lane] = wi - w;        // exclusive prefix of the waves
    if (lane == kEcWaves - 1) tmp[kEcWaves] = wi;   // block total
  }
  __syncthreads();
  const int out = tmp[wave] + incl - v;
  *total = tmp[kEcWaves];
  __syncthreads();
  return out;
}

// Per-token log-sum-exp of the logits (one wavefront per token), for the
// weights p = exp(g - lse).
__global__ __launch_bounds__(256) void lse_kernel(const float* __restrict__ logits,
                                                  float* __restrict__ lse, int T, int E) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const float* row = logits + static_cast<int64_t>(t) * E;
  float m = -INFINITY;
  for (int e = lane; e < E; e += kWave) m = fmaxf(m, row[e]);
  m = wave_max(m);
  float s = 0.f;
  for (int e = lane; e < E; e += kWave) s += expf(row[e] - m);
  s = wave_sum(s);
  if (lane == 0) lse[t] = m + logf(s);
}

// KPT > 0: thread tid owns tokens [tid * chunk, +chunk) with chunk <= KPT
// and loads their keys into registers once, all loads in flight together
// (indices clamped into the column); the radix passes and the compaction
// read the registers.  KPT = 0: every pass reads the column again.
template <int KPT>
__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(
    const float* __restrict__ logits, const float* __restrict__ lse,
    int32_t* __restrict__ ec_token, float* __restrict__ ec_w, int T, int E, int cap, int npow2) {
  __shared__ int hist[256];
  __shared__ int scan_tmp[kEcWaves + 1];
  __shared__ uint32_t s_sel[2];                  // K*, keys equal to K* to take
  __shared__ uint64_t picks[kEcMaxCap];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  auto key_of = [&](int t) { return f32_order_key(logits[static_cast<int64_t>(t) * E + e]); };
  const int chunk = (T + kEcThreads - 1) / kEcThreads;
  const int t0 = min(T, tid * chunk), t1 = min(T, t0 + chunk);
  constexpr int KR = KPT > 0 ? KPT : 1;
  uint32_t kr[KR];
  if constexpr (KPT > 0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) kr[j] = key_of(min(t0 + j, T - 1));
  }

  // 1. radix select of the cap-th largest key
  uint32_t prefix = 0;
  int need = cap;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kEcThreads) hist[i] = 0;
    __syncthreads();
    if constexpr (KPT > 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const uint32_t k = kr[j];
        // digits above this one must equal the prefix found so far
        const bool match = pass == 0 || ((k ^ prefix) >> (shift + 8)) == 0u;
        if (t0 + j < t1 && match) atomicAdd(&hist[(k >> shift) & 255u], 1);
      }
    } else {
      for (int t = tid; t < T; t += kEcThreads) {
        const uint32_t k = key_of(t);
        const bool match = pass == 0 || ((k ^ prefix) >> (shift + 8)) == 0u;
        if (match) atomicAdd(&hist[(k >> shift) & 255u], 1);
      }
    }
    __syncthreads();
    if (tid < kWave) {
      // the digit is the largest bin b whose count together with the bins
      // above it reaches `need`; lane l holds bins 255 - 4l .. 252 - 4l
      const int lane = tid;
      int h[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[q] = hist[255 - 4 * lane - q];
        sum += h[q];
      }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int n = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += n;
      }
      int cum = incl - sum, digit = -1, above = 0;   // cum: keys in the bins above
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (digit < 0 && cum + h[q] >= need) { digit = 255 - 4 * lane - q; above = cum; }
        cum += h[q];
      }
      const uint64_t found = __ballot(digit >= 0);
      if (lane == __ffsll(static_cast<unsigned long long>(found)) - 1) {
        s_sel[0] = prefix | (static_cast<uint32_t>(digit) << shift);
        s_sel[1] = static_cast<uint32_t>(need - above);
      }
    }
    __syncthreads();
    prefix = s_sel[0];
    need = static_cast<int>(s_sel[1]);
    __syncthreads();
  }
  const uint32_t kstar = prefix;
  const int take_eq = need;                      // of the keys equal to K*

  // 2. compaction in token order
  int gt = 0, eq = 0;
  if constexpr (KPT > 0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (t0 + j < t1) {
        gt += kr[j] > kstar;
        eq += kr[j] == kstar;
      }
    }
  } else {
    for (int t = t0; t < t1; ++t) {
      const uint32_t k = key_of(t);
      gt += k > kstar;
      eq += k == kstar;
    }
  }
  int tot;
  const int eq_before = block_exclusive_scan(eq, scan_tmp, &tot);
  const int my_eq = max(0, min(eq, take_eq - eq_before));
  const int pos0 = block_exclusive_scan(gt + my_eq, scan_tmp, &tot);
  for (int i = tid; i < npow2; i += kEcThreads) picks[i] = 0ull;   // sorts last
  __syncthreads();
  int pos = pos0, eq_seen = 0;
  auto place = [&](int t, uint32_t k) {
    bool take = k > kstar;
    if (k == kstar) { take = eq_seen < my_eq; ++eq_seen; }
    if (take) {
      picks[pos++] = (static_cast<uint64_t>(k) << 32) |
                     static_cast<uint64_t>(0xFFFFFFFFu - static_cast<uint32_t>(t));
    }
  };
  if constexpr (KPT > 0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (t0 + j < t1) place(t0 + j, kr[j]);
  } else {
    for (int t = t0; t < t1; ++t) place(t, key_of(t));
  }
  __syncthreads();

  // 3. bitonic sort, larger composite key first.  Up to one key per
  // thread: the key stays in a register, partners closer than a wavefront
  // are reached by shuffles and only the wider strides go through LDS.
  if (npow2 <= kEcThreads) {
    uint64_t key = tid < npow2 ? picks[tid] : 0ull;
    for (int size = 2; size <= npow2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        uint64_t other;
        if (stride >= kWave) {
          __syncthreads();                       // every read of the last round is done
          if (tid < npow2) picks[tid] = key;
          __syncthreads();
          other = tid < npow2 ? picks[tid ^ stride] : 0ull;
        } else {
          const uint32_t lo = __shfl_xor(static_cast<uint32_t>(key), stride, kWave);
          const uint32_t hi = __shfl_xor(static_cast<uint32_t>(key >> 32), stride, kWave);
          other = (static_cast<uint64_t>(hi) << 32) | lo;
        }
        // the lower index of a pair keeps the larger key in a descending
        // run, the smaller in an ascending one
        const bool desc = (tid & size) == 0;
        const bool lower = (tid & stride) == 0;
        key = (desc == lower) ? (key > other ? key : other) : (key < other ? key : other);
      }
    }
    __syncthreads();
    if (tid < npow2) picks[tid] = key;
  } else {
    for (int size = 2; size <= npow2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < npow2; i += kEcThreads) {
          const int j = i ^ stride;
          if (j > i) {
            const uint64_t a = picks[i], b = picks[j];
            const bool desc = (i & size) == 0;
            if (desc ? (a < b) : (a > b)) { picks[i] = b; picks[j] = a; }
          }
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();
  for (int j = tid; j < cap; j += kEcThreads) {
    const int t = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(picks[j]));
    const float g = logits[static_cast<int64_t>(t) * E + e];
    ec_token[static_cast<int64_t>(e) * cap + j] = t;
    ec_w[static_cast<int64_t>(e) * cap + j] = expf(g - lse[t]);
  }
}

// row_of_te := -1, w_te := 0 over [T, E].
__global__ __launch_bounds__(256) void ec_clear_kernel(int32_t* __restrict__ row_of_te,
                                                       float* __restrict__ w_te, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) { row_of_te[i] = -1; w_te[i] = 0.f; }
}

// Row r = e*cap + j holds token ec_token[r]: fill the token-major maps, the
// offsets, and gather x into x_perm (one wavefront per row, 16-byte chunks).
__global__ __launch_bounds__(256) void ec_scatter_kernel(
    const int32_t* __restrict__ ec_token, const float* __restrict__ ec_w,
    const u32x4_t* __restrict__ x, int32_t* __restrict__ offsets, int32_t* __restrict__ row_of_te,
    float* __restrict__ w_te, u32x4_t* __restrict__ x_perm, int E, int cap, int row_chunks) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= E; i += blockDim.x) offsets[i] = i * cap;
  if (r >= static_cast<int64_t>(E) * cap) return;
  const int t = ec_token[r];
  const int e = static_cast<int>(r / cap);
  if (lane == 0) {
    row_of_te[static_cast<int64_t>(t) * E + e] = static_cast<int32_t>(r);
    w_te[static_cast<int64_t>(t) * E + e] = ec_w[r];
  }
  const u32x4_t* src = x + static_cast<int64_t>(t) * row_chunks;
  u32x4_t* dst = x_perm + r * row_chunks;
  for (int c = lane; c < row_chunks; c += kWave) dst[c] = src[c];
}

}  // namespace

size_t ec_workspace_bytes(int64_t T, int64_t d, int E) {
  const size_t route = (route_workspace_bytes(T, d, E) + 255) & ~static_cast<size_t>(255);
  return route + static_cast<size_t>(T) * sizeof(float);
}

hipError_t launch_route_ec(int64_t T, int64_t d, int E, int64_t cap, bool bf16, const void* x,
                           const void* w_gate, float* logits, int32_t* ec_token, float* ec_w,
                           void* ws, hipStream_t s) {
  hipError_t err = launch_logits(T, d, E, bf16, x, w_gate, logits, ws, s);
  if (err != hipSuccess || cap == 0) return err;
  float* lse = reinterpret_cast<float*>(
      static_cast<char*>(ws) +
      ((route_workspace_bytes(T, d, E) + 255) & ~static_cast<size_t>(255)));
  hipLaunchKernelGGL(lse_kernel, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(256), 0, s,
                     logits, lse, static_cast<int>(T), E);
  int npow2 = 1;
  while (npow2 < cap) npow2 <<= 1;
  // keys per thread held in registers: 4 or 16 tokens, else none
  const int64_t chunk = (T + kEcThreads - 1) / kEcThreads;
  const dim3 grid(static_cast<unsigned>(E)), block(kEcThreads);
  const int Ti = static_cast<int>(T), capi = static_cast<int>(cap);
  if (chunk <= 4)
    hipLaunchKernelGGL(ec_select_kernel<4>, grid, block, 0, s, logits, lse, ec_token, ec_w, Ti, E,
                       capi, npow2);
  else if (chunk <= 16)
    hipLaunchKernelGGL(ec_select_kernel<16>, grid, block, 0, s, logits, lse, ec_token, ec_w, Ti,
                       E, capi, npow2);
  else
    hipLaunchKernelGGL(ec_select_kernel<0>, grid, block, 0, s, logits, lse, ec_token, ec_w, Ti, E,
                       capi, npow2);
  return hipGetLastError();
}

hipError_t launch_permute_ec(int64_t T, int64_t d, int E, int64_t cap, bool bf16,
                             const int32_t* ec_token, const float* ec_w, const void* x,
                             int32_t* offsets, int32_t* row_of_te, float* w_te, void* x_perm,
                             hipStream_t s) {
  const int64_t n = T * E;
  hipLaunchKernelGGL(ec_clear_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     s, row_of_te, w_te, n);
  const int64_t rows = static_cast<int64_t>(E) * cap;
  const int row_chunks = static_cast<int>(d * (bf16 ? 2 : 4) / 16);
  const int64_t blocks = std::max<int64_t>(1, (rows + 3) / 4);
  hipLaunchKernelGGL(ec_scatter_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     ec_token, ec_w, static_cast<const u32x4_t*>(x), offsets, row_of_te, w_te,
                     static_cast<u32x4_t*>(x_perm), E, static_cast<int>(cap), row_chunks);
  return hipGetLastError();
}

}  // namespace moe
