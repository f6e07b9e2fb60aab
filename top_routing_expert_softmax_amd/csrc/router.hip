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
// bf16 with E a multiple of 8: the matrix-core kernel router_mfma_kernel
// below (its comment has the details) computes the same logits with MFMA,
// also exactly on the dyadic grid, and runs the same epilogue; with few
// tokens it splits d over blocks in the same way and hands its partial
// logits to the same select kernel.
//
// Top-k: one wavefront per token (four tokens per wavefront when E <= 64),
// each lane holding up to four logits; k rounds of a wave-wide max of the
// logits' order keys (DPP within rows of 16 lanes, then the row maxima)
// pick the experts, larger logit first, and a ballot of the lanes holding
// that key gives the lowest index among ties; the weights are
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

// Among entries r < 4 of every lane whose key equals best (wave-uniform),
// the lowest expert index lane + 64 r.  best must be held by some entry.
__device__ __forceinline__ int lowest_holder(const uint32_t (&key)[4], uint32_t best) {
  const uint64_t m0 = __ballot(key[0] == best), m1 = __ballot(key[1] == best);
  const uint64_t m2 = __ballot(key[2] == best), m3 = __ballot(key[3] == best);
  return m0 ? __builtin_ctzll(m0)
            : m1 ? 64 + __builtin_ctzll(m1) : m2 ? 128 + __builtin_ctzll(m2) : 192 + __builtin_ctzll(m3);
}

// Top-k of one token held by one wavefront: lane holds logits of experts
// lane + 64 r (r < 4) in v[r].  Writes k ids and renormalised weights.
// Each of the k rounds takes the largest order key left (key 0 marks
// experts past E and those already taken: every finite logit has a larger
// key), then the lowest expert index holding it.
__device__ __forceinline__ void topk_select(const float (&v)[4], int E, int k, int lane,
                                            int32_t* __restrict__ idx_row,
                                            float* __restrict__ w_row) {
  uint32_t key[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) key[r] = lane + kWave * r < E ? f32_order_key(v[r]) : 0u;
  float gmax = 0.f, wsum = 0.f, my_w = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t best = wave_max_u32(max(max(key[0], key[1]), max(key[2], key[3])));
    const int e_sel = lowest_holder(key, best);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (e_sel == lane + kWave * r) key[r] = 0u;
    const float g_sel = from_order_key(best);
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

// Top-k of four tokens at once when E <= 64: lane holds the logit of
// expert lane of token r in v[r] (tokens r >= ntok do not exist and are not
// written).  The same rounds as topk_select, run for the four tokens side
// by side so that their cross-lane reductions overlap; the results are
// bit for bit those of topk_select.  Rows idx_rows + r * k, w_rows + r * k.
__device__ __forceinline__ void topk_select4(const float (&v)[4], int E, int k, int lane,
                                             int ntok, int32_t* __restrict__ idx_rows,
                                             float* __restrict__ w_rows) {
  uint32_t key[4];
  float gmax[4], wsum[4], my_w[4];
  int my_e[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    key[r] = lane < E && r < ntok ? f32_order_key(v[r]) : 0u;
    gmax[r] = 0.f; wsum[r] = 0.f; my_w[r] = 0.f; my_e[r] = 0;
  }
  for (int j = 0; j < k; ++j) {
    uint32_t best[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) best[r] = wave_max_u32(key[r]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e_sel = __builtin_ctzll(__ballot(key[r] == best[r]));
      if (e_sel == lane) key[r] = 0u;
      const float g_sel = from_order_key(best[r]);
      if (j == 0) gmax[r] = g_sel;
      const float ex = expf(g_sel - gmax[r]);
      wsum[r] += ex;
      if (lane == j) { my_w[r] = ex; my_e[r] = e_sel; }
    }
  }
  if (lane < k) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r < ntok) {
        idx_rows[r * k + lane] = my_e[r];
        w_rows[r * k + lane] = my_w[r] / wsum[r];
      }
    }
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
  // keep topk_groups groups: rounds of a wave max over the group scores
  // (key 0: not a group, or kept already), ties to the lower group
  uint64_t kept = 0;
  for (int j = 0; j < gp.topk_groups; ++j) {
    const uint32_t key = lane < gp.n_groups && !((kept >> lane) & 1ull) ? gkey : 0u;
    const uint32_t best = wave_max_u32(key);
    kept |= 1ull << __builtin_ctzll(__ballot(key == best));
  }
  // k experts of the kept groups by biased score, ties to the lower expert
  uint32_t key[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane + kWave * r;
    key[r] = e < E && ((kept >> (e / G)) & 1ull) ? f32_order_key(bsc[r]) : 0u;
  }
  float wsum = 0.f, my_s = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t best = wave_max_u32(max(max(key[0], key[1]), max(key[2], key[3])));
    const int e_sel = lowest_holder(key, best);
    // the lane that holds the winner hands its affinity to every lane
    const int r_sel = e_sel / kWave;
    const float s_own = r_sel == 0 ? s[0] : r_sel == 1 ? s[1] : r_sel == 2 ? s[2] : s[3];
    const float s_sel = __uint_as_float(
        __builtin_amdgcn_readlane(__float_as_uint(s_own), e_sel & (kWave - 1)));
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (e_sel == lane + kWave * r) key[r] = 0u;
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
// accumulators (s mod 8, splits in order) that are combined in a fixed
// order; wavefront 0 then selects from the LDS copy of the row.
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ partial, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int nT, int E, int k, int S,
    GateParams gp) {
  __shared__ float row[256];
  __shared__ float scratch[256];
  const int t = blockIdx.x;
  const int e = threadIdx.x;
  float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // split s goes to accumulator s mod 8, splits in order; the loads of 32
  // splits go out together: unconditional, at indices clamped into the
  // buffer (splits past S and experts past E add nothing)
  const int ec = min(e, E - 1);
  for (int s0 = 0; s0 < S; s0 += 32) {
    float v[32];
#pragma unroll
    for (int q = 0; q < 32; ++q)
      v[q] = partial[(static_cast<int64_t>(min(s0 + q, S - 1)) * nT + t) * E + ec];
#pragma unroll
    for (int q = 0; q < 32; ++q)
      if (e < E && s0 + q < S) s8[q % 8] += v[q];
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

// Matrix-core router (bf16, E a multiple of 8, many tokens): a block owns
// 16 * MT tokens and its nw waves split d into ranges of 32-wide k-steps.
// Each wave runs v_mfma_f32_16x16x32_bf16 with x as the A operand (lane l:
// token l % 16 of a 16-token tile, k = 8 (l / 16) .. +7, one 16-byte load)
// and W_gate as the B operand (lane l: expert 16 g + l % 16 of column group
// g, the same k).  W_gate is stored [d, E] with the experts contiguous, so
// the wave copies U k-steps of its rows into its own LDS slice and reads
// the B fragments back with LDS transpose reads.  Accumulator element v of
// lane l is token 4 (l / 16) + v of the tile.  bf16 products are exact in
// fp32, so on the dyadic input grid every MFMA sum is exact too and the
// logits equal the fp32 FMA kernel's bit for bit.  The waves' partial
// logits meet in LDS and are added in wave order; then the same top-k
// epilogue runs.  Token rows past T read row T-1 and are never stored;
// staged columns past E only feed accumulator columns that are dropped.

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

// Two LDS transpose reads (4 x 16 bit each) give one 8-value B fragment.
// In each group of 16 lanes, lane 4p+m receives in slot j element m of the
// 8 bytes that lane 4j+p addresses.  With lane 4j+p of group q pointing at
// staged row 8q+j, column c0+4p, and the second read four rows further on,
// lane i of group q holds column c0+i of rows 8q .. 8q+7.
__device__ __forceinline__ bf16x8_t read_b_frag(const char* p, int four_rows) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + four_rows));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Orders this wave's LDS accesses: the writes and reads before it are done
// before those after it (a wave's LDS operations run in issue order).
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int EP, int U>
struct MfmaRouterGeom {
  static constexpr int G = EP / 16;                  // 16-expert column groups
  static constexpr int ROWB = EP * 2 + 16;           // bytes per staged W_gate row
  static constexpr int SLICE = 32 * U * ROWB;        // one wave's staging bytes
  static constexpr int CPR = EP / 8;                 // 16-byte chunks per staged row
  static constexpr int NWC = 32 * U * CPR / kWave;   // chunk slots per lane
};

// SPLIT = true (few tokens): block (x, y) takes the k-steps
// [y * steps_per_split, +steps_per_split) of d and writes its partial logits
// to partial[y][t][e]; router_select_kernel adds the splits and selects.
template <int EP, int MT, int U, int P, bool SPLIT>
__global__ __launch_bounds__(kMaxWavesR * kWave) void router_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, float* __restrict__ partial,
    int nT, int d, int E, int k, int steps_per_split, GateParams gp) {
  using Geo = MfmaRouterGeom<EP, U>;
  constexpr int G = Geo::G, ROWB = Geo::ROWB, CPR = Geo::CPR, NWC = Geo::NWC;
  constexpr int TB = 16 * MT;
  extern __shared__ __align__(16) char smem_m[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int t0 = blockIdx.x * TB;
  const int cpe = E / 8;                       // 16-byte chunks per W_gate row
  const int nsteps = d / 32;
  const int sp0 = SPLIT ? blockIdx.y * steps_per_split : 0;
  const int sp1 = SPLIT ? min(nsteps, sp0 + steps_per_split) : nsteps;
  const int spw = (sp1 - sp0 + nw - 1) / nw;
  const int s_begin = sp0 + wave * spw;
  const int s_end = min(sp1, s_begin + spw);
  char* slice = smem_m + wave * Geo::SLICE;

  const uint16_t* xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    xrow[mt] = x + static_cast<int64_t>(min(t0 + 16 * mt + (lane & 15), nT - 1)) * d +
               8 * (lane >> 4);
  // transpose-read address of this lane in a staged k-step (column group 0)
  const int rd = (8 * (lane >> 4) + ((lane & 15) >> 2)) * ROWB + 8 * (lane & 3);

  f32x4_t acc[MT][G];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int g = 0; g < G; ++g) acc[mt][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // P k-steps per batch are loaded at once (sub-batch by sub-batch, so the
  // first can be staged while the rest are in flight), then staged and
  // multiplied U steps at a time.  Every load is unconditional and in
  // bounds: steps past the wave's range read the last step or row of d,
  // chunks past E re-read the row's last chunk; what they bring is staged
  // but never multiplied (steps) or only reaches dropped columns (chunks).
  constexpr int NB = P / U;
  for (int s = s_begin; s < s_end; s += P) {
    const int cnt = min(P, s_end - s);         // k-steps in this batch
    u32x4_t xa[MT][P];
    u32x4_t wa[NB][NWC];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int u = b * U; u < b * U + U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          xa[mt][u] = *reinterpret_cast<const u32x4_t*>(xrow[mt] + min(s + u, nsteps - 1) * 32);
      // chunk slot c = lane + 64 i: staged row c / CPR, 16-byte column c % CPR
#pragma unroll
      for (int i = 0; i < NWC; ++i) {
        const int c = lane + kWave * i, r = c / CPR, cc = min(c % CPR, cpe - 1);
        const int row = min((s + b * U) * 32 + r, d - 1);
        wa[b][i] = *reinterpret_cast<const u32x4_t*>(wg + static_cast<int64_t>(row) * E + cc * 8);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      wave_lds_order();                        // the previous sub-batch's reads are done
#pragma unroll
      for (int i = 0; i < NWC; ++i) {
        const int c = lane + kWave * i;
        *reinterpret_cast<u32x4_t*>(slice + (c / CPR) * ROWB + (c % CPR) * 16) = wa[b][i];
      }
      wave_lds_order();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // steps past the range multiply a zero A operand (the staged rows
        // there are finite W_gate rows, so they add exact zeros)
        const u32x4_t a = b * U + u < cnt ? xa[0][b * U + u] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const bf16x8_t bf = read_b_frag(slice + u * 32 * ROWB + rd + 32 * g, 4 * ROWB);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const u32x4_t am = mt == 0 ? a : (b * U + u < cnt ? xa[mt][b * U + u]
                                                               : u32x4_t{0u, 0u, 0u, 0u});
            acc[mt][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, am), bf, acc[mt][g], 0, 0, 0);
          }
        }
      }
    }
  }

  // partial logits of every wave, red[w][t][e] (over the staging slices)
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem_m);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        red[(wave * TB + 16 * mt + 4 * (lane >> 4) + v) * EP + 16 * g + (lane & 15)] =
            acc[mt][g][v];
  __syncthreads();
  // sum in wave order into red[0] (each element read and written by one
  // thread), store the logits (or this split's partial logits)
  float* dst = SPLIT ? partial + static_cast<int64_t>(blockIdx.y) * nT * E : logits;
  for (int q = threadIdx.x; q < TB * EP; q += blockDim.x) {
    float sum = red[q];
    for (int w = 1; w < nw; ++w) sum += red[w * TB * EP + q];
    red[q] = sum;
    const int t = q / EP, e = q % EP;
    if (t0 + t < nT && e < E) dst[static_cast<int64_t>(t0 + t) * E + e] = sum;
  }
  if (SPLIT || gp.v3 == 2) return;
  __syncthreads();
  if (gp.v3 == 0 && E <= kWave) {
    // four tokens per wavefront
    for (int tt = 4 * wave; tt < TB; tt += 4 * nw) {
      const int ntok = min(4, nT - (t0 + tt));
      if (ntok <= 0) break;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = lane < E ? red[(tt + r) * EP + lane] : 0.f;
      topk_select4(v, E, k, lane, ntok, topk_idx + static_cast<int64_t>(t0 + tt) * k,
                   topk_w + static_cast<int64_t>(t0 + tt) * k);
    }
    return;
  }
  for (int tt = wave; tt < TB; tt += nw) {
    const int t = t0 + tt;
    if (t >= nT) break;
    const float* row = red + tt * EP;
    if (gp.v3 == 1) {
      // E floats of scratch per wave past the summed rows (nw >= 2 leaves
      // (nw - 1) * TB * EP free floats there)
      v3_select(row, red + TB * EP + wave * EP, gp, E, k, lane,
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

// Matrix-core router plan: EP = E rounded up to a power of two (at least
// 16), 32 tokens per block once that still gives 256 blocks, U k-steps
// staged per batch (fewer for wide E, so a wave's slice stays small), and
// enough waves (d-ranges) per block to put about 2048 waves on the chip,
// within 64 KB of LDS.  With few tokens (max_splits > 1, the split count the
// workspace holds) d is also split over blocks: S <= max_splits splits of
// whole k-steps, aiming at 256 blocks.
struct MfmaRouterPlan {
  int EP, MT, U, nw, nblocks;
  int S, sps;             // d-splits and k-steps per split (S = 1: no split)
  size_t lds;
};

bool mfma_router_applies(int E, bool bf16) { return bf16 && E % 8 == 0; }

MfmaRouterPlan plan_mfma_router(int64_t T, int64_t d, int E, int max_splits) {
  MfmaRouterPlan p;
  p.EP = 16;
  while (p.EP < E) p.EP <<= 1;
  p.MT = max_splits == 1 && (T + 31) / 32 >= 256 ? 2 : 1;
  p.U = p.EP <= 32 ? 4 : (p.EP == 64 ? 2 : 1);
  const int TB = 16 * p.MT;
  p.nblocks = static_cast<int>((T + TB - 1) / TB);
  const int nsteps = static_cast<int>(d / 32);
  p.S = 1;
  p.sps = nsteps;
  if (max_splits > 1) {
    const int want = std::max(1, std::min(max_splits, (256 + p.nblocks - 1) / p.nblocks));
    p.sps = (nsteps + want - 1) / want;
    p.S = (nsteps + p.sps - 1) / p.sps;
  }
  const size_t slice = static_cast<size_t>(32) * p.U * (p.EP * 2 + 16);
  const size_t per_wave = std::max(slice, static_cast<size_t>(TB) * p.EP * 4);
  int nw = (2048 + p.nblocks * p.S - 1) / (p.nblocks * p.S);
  nw = std::min(nw, kMaxWavesR);
  nw = std::min(nw, p.sps);
  nw = std::min(nw, static_cast<int>(65536 / per_wave));
  p.nw = std::max(nw, 2);
  p.lds = per_wave * p.nw;
  return p;
}

template <int EP, int MT>
hipError_t launch_mfma_mt(const MfmaRouterPlan& p, int64_t T, int64_t d, int E, int k,
                          const void* x, const void* wg, float* logits, int32_t* idx, float* w,
                          float* partial, const GateParams& gp, hipStream_t s) {
  constexpr int U = EP <= 32 ? 4 : (EP == 64 ? 2 : 1);
  // k-steps loaded per batch: what about 200 VGPRs hold next to the
  // accumulators
  constexpr int P = EP == 16 ? 16 : EP == 32 ? 8 : EP == 64 ? 6 : EP == 128 ? 3 : (MT == 1 ? 2 : 1);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* wb = static_cast<const uint16_t*>(wg);
  if (p.S == 1) {
    hipLaunchKernelGGL((router_mfma_kernel<EP, MT, U, P, false>), dim3(p.nblocks),
                       dim3(p.nw * kWave), p.lds, s, xb, wb, logits, idx, w, nullptr,
                       static_cast<int>(T), static_cast<int>(d), E, k, p.sps, gp);
    return hipGetLastError();
  }
  if constexpr (MT == 1) {
    hipLaunchKernelGGL((router_mfma_kernel<EP, 1, U, P, true>), dim3(p.nblocks, p.S),
                       dim3(p.nw * kWave), p.lds, s, xb, wb, logits, idx, w, partial,
                       static_cast<int>(T), static_cast<int>(d), E, k, p.sps, gp);
    hipLaunchKernelGGL(router_select_kernel, dim3(static_cast<unsigned>(T)), dim3(256), 0, s,
                       partial, logits, idx, w, static_cast<int>(T), E, k, p.S, gp);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;                   // the plan splits only with MT = 1
}

template <int EP>
hipError_t launch_mfma_ep(const MfmaRouterPlan& p, int64_t T, int64_t d, int E, int k,
                          const void* x, const void* wg, float* logits, int32_t* idx, float* w,
                          float* partial, const GateParams& gp, hipStream_t s) {
  if (p.MT == 2) return launch_mfma_mt<EP, 2>(p, T, d, E, k, x, wg, logits, idx, w, partial, gp, s);
  return launch_mfma_mt<EP, 1>(p, T, d, E, k, x, wg, logits, idx, w, partial, gp, s);
}

hipError_t launch_mfma_router(int64_t T, int64_t d, int E, int k, const void* x, const void* wg,
                              float* logits, int32_t* idx, float* w, float* partial,
                              const GateParams& gp, hipStream_t s) {
  const MfmaRouterPlan p = plan_mfma_router(T, d, E, plan_router(T, d, E).S);
  switch (p.EP) {
    case 16: return launch_mfma_ep<16>(p, T, d, E, k, x, wg, logits, idx, w, partial, gp, s);
    case 32: return launch_mfma_ep<32>(p, T, d, E, k, x, wg, logits, idx, w, partial, gp, s);
    case 64: return launch_mfma_ep<64>(p, T, d, E, k, x, wg, logits, idx, w, partial, gp, s);
    case 128: return launch_mfma_ep<128>(p, T, d, E, k, x, wg, logits, idx, w, partial, gp, s);
    default: return launch_mfma_ep<256>(p, T, d, E, k, x, wg, logits, idx, w, partial, gp, s);
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
  if (mfma_router_applies(E, bf16))
    return launch_mfma_router(T, d, E, k, x, w_gate, logits, topk_idx, topk_w, partial, gp, s);
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
