// Expert FFN of decode-sized segments: weight streaming.
//
// In a decode step each touched expert sees only a few tokens while all of
// its weights are read ("CMU 11-868 Lecture 17", section 1.4: with a batch
// of 64 tokens DeepSeek-V3 touches about 222 of 256 experts, two tokens
// each), so the expert FFN is bound by HBM bandwidth.  Here every weight
// byte is read once, straight from HBM into registers, and goes through
// v_mfma_f32_16x16x32_bf16 against the segment's (at most 64) token rows;
// the matrix unit has time to spare, so no LDS staging is needed.
//
// Work split.  A block of 4 wavefronts owns one group of weight rows of one
// segment: phase 1 takes 16 rows of W1 and the same 16 rows of W3 (16
// columns of H), phase 2 takes 32 rows of W2 (32 output columns; FP8: 64).
// Its waves take the contracted dimension's batches of K
// steps round robin, so at any moment they read adjacent pieces of every
// weight row, starting at a per-block rotation of the batch order so that
// concurrent blocks read different parts of their rows; the four partial
// sums meet in LDS and are added in wave order (deterministic), then phase
// 1 applies SiLU(gate) * up and rounds H to bf16.  Segments of a few rows first copy their token rows into the
// LDS (stage_rows).
//
// Fragments (16 x 16 x 32 MFMA, lane l): the A operand holds token
// l % 16 of a 16-token group and the B operand weight row l % 16 of a
// 16-row group, both for contracted indices 8 * (l / 16) .. +7 of a 32-wide
// step; accumulator element v of lane l is token 4 * (l / 16) + v, weight
// row l % 16.  Token rows past the segment read its last row; their sums
// are never stored.
//
// FP8 weights (OCP E4M3 codes with one fp32 scale per weight row; the
// pages name FP8 expert storage, "CMU 11-868 Lecture 17" section 1.4, but
// no encoding): a lane loads 16 codes (16 consecutive contracted indices of
// a 64-wide step), converts them to bf16 in registers (exact: every E4M3
// value is a bf16 value) and feeds two MFMAs, the A operand taking the
// same 16 indices of the token rows.  The row scale multiplies the summed
// dot product (s * sum_k x_k q_k = sum_k x_k (s q_k)).  Half the bytes of
// the bf16 weights cross HBM.
#include <algorithm>
#include <atomic>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSWaves = 4;               // waves per block (K quarters)
constexpr int kSNB = 2;                  // 16-row weight fragments per K step (bf16)
constexpr int kSNB8 = 4;                 // fragments per K step (FP8, phase 2)
constexpr int kSNB8P1 = 2;               // fragments per K step (FP8, phase 1): gate, up
constexpr int kSU = 4;                   // 32-wide K steps per load batch (bf16, 16 tokens)
constexpr int kSU8 = 2;                  // 64-wide K steps per load batch (FP8 phase 2, 16 tokens)
constexpr int kSU8P1 = 4;                // the same, FP8 phase 1

struct StreamArgs {
  const void* x_perm;
  const void* x;
  const int32_t* offsets;
  const void* w1;
  const void* w3;
  const void* w2;
  const void* ws1;
  const void* ws3;
  const void* ws2;
  void* H;
  void* y_perm;
  void* y_shared;
  const float* sc1;       // FP8 row scales: [E, F] for W1 / W3, [E, d] for W2
  const float* sc3;
  const float* sc2;
  const float* ssc1;      // shared experts' scales, same layouts
  const float* ssc3;
  const float* ssc2;
  int T, d, E, Es, k, F;
  int xs_rows;            // segments of at most this many rows stage them in LDS
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Eight E4M3 codes (two words, lowest byte first) as eight bf16 values.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w0), 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w0), 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w1), 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w1), 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// SiLU with the hardware reciprocal, as in the grouped GEMM's epilogue.
__device__ __forceinline__ float silu_s(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Each block walks its K batches from a rotated start: batch b of the
// round-robin order reads physical batch (b + rot) mod nbt, rot a hash of
// the block's indices.  In unrotated order every block of a launch starts
// at K = 0 and they move through K at about the same pace, so the blocks in
// flight all read the same narrow column range of their weight rows at
// once; the rotation spreads them over the whole row (DeepSeek-V3 decode
// step: bf16 weights 3.31 -> 3.18 ms, FP8 1.733 -> 1.707 ms).  The per-block sum order
// changes with it, fixed for a given launch shape, so results stay
// deterministic.
__device__ __forceinline__ int batch_rotation(int nbt) {
  const unsigned h = (blockIdx.x * 2654435761u + blockIdx.y * 40503u) >> 7;
  return nbt > 0 ? static_cast<int>(h % static_cast<unsigned>(nbt)) : 0;
}
// first K step of round-robin batch b (b < nbt, rot < nbt)
__device__ __forceinline__ int batch_step(int b, int rot, int nbt, int U) {
  const int p = b + rot;
  return (p < nbt ? p : p - nbt) * U;
}

// The segment's token rows (rows x K bf16) copied into the LDS, row r at
// element r * (K + 8): the 16-byte pad puts the rows of a fragment read on
// different banks.  A decode segment holds a few tokens, so every lane of
// an A-operand load addresses one of a few rows; from L2 those loads cost
// about as many requests as the weight stream, and from LDS none.  Direct-
// to-LDS loads of 16 bytes, 64 pieces per wave instruction (the pad pieces
// load the first piece again); every wave waits for its loads, then the
// block meets at a barrier.
__device__ __forceinline__ void stage_rows(const uint16_t* A, int rows, int K, uint16_t* xs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int per_row = (K + 8) / 8;                 // 16-byte pieces per LDS row
  const int total = rows * per_row;
  for (int j = wave; j * kWave < total; j += kSWaves) {
    const int p = j * kWave + lane;
    const int r = p / per_row, c = p - r * per_row;
    const uint16_t* src = c < K / 8 ? A + static_cast<int64_t>(r) * K + c * 8 : A;
    if (p < total)
      __builtin_amdgcn_global_load_lds(src, reinterpret_cast<uint32_t*>(xs + j * kWave * 8), 16,
                                       0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0xF70);               // vmcnt(0)
  __syncthreads();
}

// Sum the four quarters of a block in wave order, one token group at a
// time (wave tg % 4 finishes group tg), scale (FP8) and store.
template <int PHASE, int TG, bool FP8, int NB>
__device__ __forceinline__ void stream_finish(const StreamArgs& a, f32x4_t (&acc)[TG][NB],
                                              int seg, int rows, int arow0, int hrow0, int n0,
                                              float* red) {
  // Phase 1: fragments b < NB/2 hold gate (W1) rows n0 + 16 b, the others
  // the same rows of W3.  Phase 2: fragment b holds W2 rows n0 + 16 b.
  const bool routed = seg < a.E;
  const int e = routed ? seg : seg - a.E;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  float scale[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    scale[b] = 1.0f;
    if (FP8) {
      if (PHASE == 1) {
        const int64_t at = static_cast<int64_t>(e) * a.F + n0 + 16 * (b % (NB / 2)) + (lane & 15);
        scale[b] = b < NB / 2 ? (routed ? a.sc1 : a.ssc1)[at] : (routed ? a.sc3 : a.ssc3)[at];
      } else {
        scale[b] = (routed ? a.sc2 : a.ssc2)[static_cast<int64_t>(e) * a.d + n0 + b * 16 +
                                             (lane & 15)];
      }
    }
  }
  f32x4_t* R = reinterpret_cast<f32x4_t*>(red);
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
#pragma unroll
    for (int b = 0; b < NB; ++b) R[(wave * NB + b) * kWave + lane] = acc[tg][b];
    __syncthreads();
    if (wave == (tg & (kSWaves - 1))) {
      f32x4_t v[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        v[b] = R[b * kWave + lane];
#pragma unroll
        for (int w = 1; w < kSWaves; ++w) v[b] += R[(w * NB + b) * kWave + lane];
        v[b] *= scale[b];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = tg * 16 + 4 * (lane >> 4) + q;
        if (m >= rows) continue;
        if (PHASE == 1) {
          uint16_t* Hout = static_cast<uint16_t*>(a.H) + static_cast<int64_t>(hrow0 + m) * a.F;
#pragma unroll
          for (int b = 0; b < NB / 2; ++b)
            Hout[n0 + 16 * b + (lane & 15)] = f32_to_bf16(silu_s(v[b][q]) * v[b + NB / 2][q]);
        } else {
          uint16_t* Y = routed
              ? static_cast<uint16_t*>(a.y_perm) + static_cast<int64_t>(arow0 + m) * a.d
              : static_cast<uint16_t*>(a.y_shared) +
                    static_cast<int64_t>(hrow0 - a.T * a.k + m) * a.d;
#pragma unroll
          for (int b = 0; b < NB; ++b) Y[n0 + b * 16 + (lane & 15)] = f32_to_bf16(v[b][q]);
        }
      }
    }
    __syncthreads();
  }
}

// One block, TG groups of 16 tokens.  U = K steps loaded per batch.
template <int PHASE, int TG, bool XS>
__device__ __forceinline__ void stream_block(const StreamArgs& a, int seg, int rows, int arow0,
                                             int hrow0, float* red, uint16_t* xs) {
  constexpr int U = TG == 1 ? kSU : (TG == 2 ? (kSU + 1) / 2 : 1);
  const bool routed = seg < a.E;
  const int e = routed ? seg : seg - a.E;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int K = PHASE == 1 ? a.d : a.F;
  const int64_t wstride = static_cast<int64_t>(a.F) * a.d;

  // weight rows of the two B fragments
  const uint16_t* wrow[kSNB];
  int n0;
  if (PHASE == 1) {
    n0 = blockIdx.x * 16;                      // H columns n0 .. n0+15
    const uint16_t* W1 = static_cast<const uint16_t*>(routed ? a.w1 : a.ws1) + e * wstride;
    const uint16_t* W3 = static_cast<const uint16_t*>(routed ? a.w3 : a.ws3) + e * wstride;
    wrow[0] = W1 + static_cast<int64_t>(n0 + (lane & 15)) * K;
    wrow[1] = W3 + static_cast<int64_t>(n0 + (lane & 15)) * K;
  } else {
    n0 = blockIdx.x * 32;                      // output columns n0 .. n0+31
    const uint16_t* W2 = static_cast<const uint16_t*>(routed ? a.w2 : a.ws2) + e * wstride;
    wrow[0] = W2 + static_cast<int64_t>(n0 + (lane & 15)) * K;
    wrow[1] = W2 + static_cast<int64_t>(n0 + 16 + (lane & 15)) * K;
  }
  // token rows of the TG A fragments
  const uint16_t* arow[TG];
  const uint16_t* Abase = PHASE == 1
      ? static_cast<const uint16_t*>(routed ? a.x_perm : a.x) + static_cast<int64_t>(arow0) * K
      : static_cast<const uint16_t*>(a.H) + static_cast<int64_t>(hrow0) * K;
  if constexpr (XS) {
    stage_rows(Abase, rows, K, xs);
    arow[0] = xs + min(lane & 15, rows - 1) * (K + 8);
  } else {
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const int m = min(tg * 16 + (lane & 15), rows - 1);
      arow[tg] = Abase + static_cast<int64_t>(m) * K;
    }
  }
  const int kq = 8 * (lane >> 4);

  f32x4_t acc[TG][kSNB];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int b = 0; b < kSNB; ++b) acc[tg][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The 32-wide K steps go to the waves in batches of U, round robin (as in
  // stream_block_fp8), from the block's rotated start (batch_step); the
  // steps past the whole batches go to wave (whole batches) % 4.
  const int nsteps = K / 32;
  const int nbt = nsteps / U;
  const int nbw = nbt > wave ? (nbt - wave + kSWaves - 1) / kSWaves : 0;
  const int rot = batch_rotation(nbt);
#define MOE_SLOAD(FA, FB, S0)                                                              \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                                         \
    const int kk = ((S0) + u) * 32 + kq;                                                  \
    _Pragma("unroll") for (int b = 0; b < kSNB; ++b)                                      \
      FB[u][b] = *reinterpret_cast<const bf16x8_t*>(wrow[b] + kk);                        \
    _Pragma("unroll") for (int tg = 0; tg < TG; ++tg)                                     \
      FA[u][tg] = *reinterpret_cast<const bf16x8_t*>(arow[tg] + kk);                      \
  }
#define MOE_SMFMA(FA, FB)                                                                  \
  _Pragma("unroll") for (int u = 0; u < U; ++u)                                           \
    _Pragma("unroll") for (int tg = 0; tg < TG; ++tg)                                     \
      _Pragma("unroll") for (int b = 0; b < kSNB; ++b)                                    \
        acc[tg][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(FA[u][tg], FB[u][b], acc[tg][b], 0, 0, 0);
  int j = 0;
  if (nbw >= 2) {
    bf16x8_t fa0[U][TG], fb0[U][kSNB], fa1[U][TG], fb1[U][kSNB];
    MOE_SLOAD(fa0, fb0, batch_step(wave, rot, nbt, U));
    j = 1;
    for (; j + 2 <= nbw; j += 2) {
      MOE_SLOAD(fa1, fb1, batch_step(wave + kSWaves * j, rot, nbt, U));
      MOE_SMFMA(fa0, fb0);
      MOE_SLOAD(fa0, fb0, batch_step(wave + kSWaves * (j + 1), rot, nbt, U));
      MOE_SMFMA(fa1, fb1);
    }
    MOE_SMFMA(fa0, fb0);
  }
  for (; j < nbw; ++j) {
    bf16x8_t fa[U][TG], fb[U][kSNB];
    MOE_SLOAD(fa, fb, batch_step(wave + kSWaves * j, rot, nbt, U));
    MOE_SMFMA(fa, fb);
  }
#undef MOE_SLOAD
#undef MOE_SMFMA
  const bool tailw = wave == nbt % kSWaves;
  const int s1 = tailw ? nsteps : 0;
  for (int s = nbt * U; s < s1; ++s) {
    const int kk = s * 32 + kq;
    bf16x8_t fb[kSNB], fa[TG];
#pragma unroll
    for (int b = 0; b < kSNB; ++b)
      fb[b] = *reinterpret_cast<const bf16x8_t*>(wrow[b] + kk);
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) fa[tg] = *reinterpret_cast<const bf16x8_t*>(arow[tg] + kk);
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int b = 0; b < kSNB; ++b)
        acc[tg][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[tg], fb[b], acc[tg][b], 0, 0, 0);
  }

  stream_finish<PHASE, TG, false, kSNB>(a, acc, seg, rows, arow0, hrow0, n0, red);
}

// FP8 weights: as stream_block, on 64-wide K steps of E4M3 codes.
template <int PHASE, int TG, bool XS>
__device__ __forceinline__ void stream_block_fp8(const StreamArgs& a, int seg, int rows,
                                                 int arow0, int hrow0, float* red,
                                                 uint16_t* xs) {
  // Phase 1 (rows of d codes): a wave's batch covers 256 bytes of each of
  // 32 weight rows (two fragments, four 64-wide steps), the shape of the
  // bf16 kernel's batches.  Four fragments of two steps (128 bytes of each
  // of 64 rows, the same registers) measured 1.707 ms against 1.622 ms on
  // the DeepSeek-V3 decode step: longer pieces of fewer rows at a time
  // stream faster.  Phase 2 (rows of F = 2048 codes) keeps four fragments
  // of two steps, which leaves each wave four batches to pipeline.
  constexpr int NB = PHASE == 1 ? kSNB8P1 : kSNB8;
  constexpr int U = TG == 1 ? (PHASE == 1 ? kSU8P1 : kSU8) : 1;   // 64-wide K steps per batch
  const bool routed = seg < a.E;
  const int e = routed ? seg : seg - a.E;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int K = PHASE == 1 ? a.d : a.F;
  const int64_t wstride = static_cast<int64_t>(a.F) * a.d;     // codes per expert matrix

  const uint8_t* wrow[NB];
  int n0;
  if (PHASE == 1) {
    n0 = blockIdx.x * 8 * NB;                    // NB/2 gate and NB/2 up fragments
    const uint8_t* W1 = static_cast<const uint8_t*>(routed ? a.w1 : a.ws1) + e * wstride;
    const uint8_t* W3 = static_cast<const uint8_t*>(routed ? a.w3 : a.ws3) + e * wstride;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      wrow[b] = (b < NB / 2 ? W1 : W3) +
                static_cast<int64_t>(n0 + 16 * (b % (NB / 2)) + (lane & 15)) * K;
  } else {
    n0 = blockIdx.x * 16 * NB;
    const uint8_t* W2 = static_cast<const uint8_t*>(routed ? a.w2 : a.ws2) + e * wstride;
#pragma unroll
    for (int b = 0; b < NB; ++b) wrow[b] = W2 + static_cast<int64_t>(n0 + 16 * b + (lane & 15)) * K;
  }
  const uint16_t* arow[TG];
  const uint16_t* Abase = PHASE == 1
      ? static_cast<const uint16_t*>(routed ? a.x_perm : a.x) + static_cast<int64_t>(arow0) * K
      : static_cast<const uint16_t*>(a.H) + static_cast<int64_t>(hrow0) * K;
  if constexpr (XS) {
    stage_rows(Abase, rows, K, xs);
    arow[0] = xs + min(lane & 15, rows - 1) * (K + 8);
  } else {
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const int m = min(tg * 16 + (lane & 15), rows - 1);
      arow[tg] = Abase + static_cast<int64_t>(m) * K;
    }
  }
  const int kq = 16 * (lane >> 4);       // the lane's 16 indices of a 64-wide step

  f32x4_t acc[TG][NB];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[tg][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The K steps go to the waves in batches of U, round robin: wave w takes
  // batches w, w + 4, ..., so the four waves of a block read adjacent
  // pieces of every weight row at the same moment (rows of d = 7168 codes
  // are read front to back once, not in four far-apart streams); the steps
  // past the whole batches go to wave (whole batches) % 4.  The batch
  // order starts at a per-block rotation (batch_step).
  const int nsteps = K / 64;
  const int nbt = nsteps / U;
  const int nbw = nbt > wave ? (nbt - wave + kSWaves - 1) / kSWaves : 0;
  const int rot = batch_rotation(nbt);
#define MOE_FLOAD(FQ, FA, S0)                                                              \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                                         \
    const int kk = ((S0) + u) * 64 + kq;                                                  \
    _Pragma("unroll") for (int b = 0; b < NB; ++b)                                      \
      FQ[u][b] = *reinterpret_cast<const u32x4_t*>(wrow[b] + kk);                         \
    _Pragma("unroll") for (int tg = 0; tg < TG; ++tg) {                                   \
      FA[u][tg][0] = *reinterpret_cast<const bf16x8_t*>(arow[tg] + kk);                   \
      FA[u][tg][1] = *reinterpret_cast<const bf16x8_t*>(arow[tg] + kk + 8);               \
    }                                                                                      \
  }
#define MOE_FMFMA(FQ, FA)                                                                  \
  _Pragma("unroll") for (int u = 0; u < U; ++u)                                           \
    _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                    \
      const bf16x8_t lo = e4m3x8_to_bf16(FQ[u][b][0], FQ[u][b][1]);                       \
      const bf16x8_t hi = e4m3x8_to_bf16(FQ[u][b][2], FQ[u][b][3]);                       \
      _Pragma("unroll") for (int tg = 0; tg < TG; ++tg) {                                 \
        acc[tg][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(FA[u][tg][0], lo, acc[tg][b], \
                                                              0, 0, 0);                    \
        acc[tg][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(FA[u][tg][1], hi, acc[tg][b], \
                                                              0, 0, 0);                    \
      }                                                                                    \
    }
  int j = 0;
  if (nbw >= 2) {
    // two batches in flight: load batch j+1, then use batch j
    u32x4_t q0[U][NB], q1[U][NB];
    bf16x8_t x0[U][TG][2], x1[U][TG][2];
    MOE_FLOAD(q0, x0, batch_step(wave, rot, nbt, U));
    j = 1;
    for (; j + 2 <= nbw; j += 2) {
      MOE_FLOAD(q1, x1, batch_step(wave + kSWaves * j, rot, nbt, U));
      MOE_FMFMA(q0, x0);
      MOE_FLOAD(q0, x0, batch_step(wave + kSWaves * (j + 1), rot, nbt, U));
      MOE_FMFMA(q1, x1);
    }
    MOE_FMFMA(q0, x0);
  }
  for (; j < nbw; ++j) {
    u32x4_t q[U][NB];
    bf16x8_t xa[U][TG][2];
    MOE_FLOAD(q, xa, batch_step(wave + kSWaves * j, rot, nbt, U));
    MOE_FMFMA(q, xa);
  }
  if constexpr (U > 1) {
    if (wave == nbt % kSWaves) {
      for (int s = nbt * U; s < nsteps; ++s) {
        u32x4_t q[1][NB];
        bf16x8_t xa[1][TG][2];
        {
          const int kk = s * 64 + kq;
#pragma unroll
          for (int b = 0; b < NB; ++b) q[0][b] = *reinterpret_cast<const u32x4_t*>(wrow[b] + kk);
#pragma unroll
          for (int tg = 0; tg < TG; ++tg) {
            xa[0][tg][0] = *reinterpret_cast<const bf16x8_t*>(arow[tg] + kk);
            xa[0][tg][1] = *reinterpret_cast<const bf16x8_t*>(arow[tg] + kk + 8);
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const bf16x8_t lo = e4m3x8_to_bf16(q[0][b][0], q[0][b][1]);
          const bf16x8_t hi = e4m3x8_to_bf16(q[0][b][2], q[0][b][3]);
#pragma unroll
          for (int tg = 0; tg < TG; ++tg) {
            acc[tg][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[0][tg][0], lo, acc[tg][b], 0, 0, 0);
            acc[tg][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[0][tg][1], hi, acc[tg][b], 0, 0, 0);
          }
        }
      }
    }
  }
#undef MOE_FLOAD
#undef MOE_FMFMA
  stream_finish<PHASE, TG, true, NB>(a, acc, seg, rows, arow0, hrow0, n0, red);
}

// Grid: x = weight-row group, y = segment (shared experts, then routed).
// Segments with no rows, or more than kStreamMaxRows rows, exit at once.
template <int PHASE, bool FP8>
__global__ __launch_bounds__(kSWaves * kWave) void ffn_stream_kernel(StreamArgs a) {
  static_assert(kSNB8 >= kSNB8P1, "the reduction buffer holds the larger FP8 block");
  __shared__ f32x4_t red[kSWaves * (FP8 ? kSNB8 : kSNB) * kWave];
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // a.xs_rows x (K + 8)
  // the shared experts first: their blocks carry all T tokens, run longest
  // and would otherwise form the launch's tail
  const int y = static_cast<int>(blockIdx.y);
  const int seg = y < a.Es ? a.E + y : y - a.Es;
  int rows, arow0, hrow0;
  if (seg < a.E) {
    arow0 = a.offsets[seg];
    rows = a.offsets[seg + 1] - arow0;
    hrow0 = arow0;
  } else {
    arow0 = 0;
    rows = a.T;
    hrow0 = a.T * a.k + (seg - a.E) * a.T;
  }
  if (rows <= 0 || rows > kStreamMaxRows) return;
  float* r = reinterpret_cast<float*>(red);
  if constexpr (FP8) {
    if (rows <= a.xs_rows) {
      stream_block_fp8<PHASE, 1, true>(a, seg, rows, arow0, hrow0, r, xs);
      return;
    }
    switch ((rows + 15) / 16) {
      case 1: stream_block_fp8<PHASE, 1, false>(a, seg, rows, arow0, hrow0, r, xs); break;
      case 2: stream_block_fp8<PHASE, 2, false>(a, seg, rows, arow0, hrow0, r, xs); break;
      case 3: stream_block_fp8<PHASE, 3, false>(a, seg, rows, arow0, hrow0, r, xs); break;
      default: stream_block_fp8<PHASE, 4, false>(a, seg, rows, arow0, hrow0, r, xs); break;
    }
  } else {
    if (rows <= a.xs_rows) {
      stream_block<PHASE, 1, true>(a, seg, rows, arow0, hrow0, r, xs);
      return;
    }
    switch ((rows + 15) / 16) {
      case 1: stream_block<PHASE, 1, false>(a, seg, rows, arow0, hrow0, r, xs); break;
      case 2: stream_block<PHASE, 2, false>(a, seg, rows, arow0, hrow0, r, xs); break;
      case 3: stream_block<PHASE, 3, false>(a, seg, rows, arow0, hrow0, r, xs); break;
      default: stream_block<PHASE, 4, false>(a, seg, rows, arow0, hrow0, r, xs); break;
    }
  }
}

// Dynamic LDS above the default limit is a per-device setting of a
// kernel: raise it once for each (kernel, device); sizes within the
// default need nothing.
template <auto Kern>
hipError_t allow_stream_lds(size_t bytes) {
  if (bytes <= 48 * 1024) return hipSuccess;
  static std::atomic<uint64_t> done{0};        // one bit per device id < 64
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  err = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 60 * 1024);
  if (err == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
  return err;
}

}  // namespace

hipError_t launch_ffn_stream(int phase, int64_t T, int64_t d, int E, int E_shared, int k,
                             int64_t F, const void* x_perm, const int32_t* offsets,
                             const void* x, const void* w1, const void* w3, const void* w2,
                             const void* ws1, const void* ws3, const void* ws2, void* H,
                             void* y_perm, void* y_shared, hipStream_t s, const float* sc1,
                             const float* sc3, const float* sc2, const float* ssc1,
                             const float* ssc3, const float* ssc2) {
  StreamArgs a{x_perm, x, offsets, w1, w3, w2, ws1, ws3, ws2, H, y_perm, y_shared,
               sc1, sc3, sc2, ssc1, ssc3, ssc2,
               static_cast<int>(T), static_cast<int>(d), E, E_shared, k, static_cast<int>(F),
               0};
  const bool fp8 = sc1 != nullptr;
  const unsigned nseg = static_cast<unsigned>(E + E_shared);
  const dim3 block(kSWaves * kWave);
  // H columns per block: 8 * fragments (half gate, half up); output
  // columns per block: 16 * fragments
  const int nb = fp8 ? (phase == 1 ? kSNB8P1 : kSNB8) : kSNB;
  // Token rows staged in LDS for segments of up to 4 (FP8) or 3 (bf16)
  // rows, within 60 KB or 45 KB: two FP8 blocks (216 registers a lane) or
  // three bf16 blocks (144) still fit a compute unit's 160 KB.
  const int64_t K = phase == 1 ? d : F;
  const int64_t row_bytes = (K + 8) * 2;
  a.xs_rows = static_cast<int>(std::min<int64_t>(fp8 ? 4 : 3, (fp8 ? 60 : 45) * 1024 / row_bytes));
  const size_t lds = static_cast<size_t>(a.xs_rows * row_bytes);
  hipError_t err = hipSuccess;
  if (phase == 1) {
    const dim3 grid(static_cast<unsigned>(F / (8 * nb)), nseg);
    if (fp8) {
      err = allow_stream_lds<ffn_stream_kernel<1, true>>(lds);
      if (err == hipSuccess) hipLaunchKernelGGL((ffn_stream_kernel<1, true>), grid, block, lds, s, a);
    } else {
      err = allow_stream_lds<ffn_stream_kernel<1, false>>(lds);
      if (err == hipSuccess) hipLaunchKernelGGL((ffn_stream_kernel<1, false>), grid, block, lds, s, a);
    }
  } else {
    const dim3 grid(static_cast<unsigned>(d / (16 * nb)), nseg);
    if (fp8) {
      err = allow_stream_lds<ffn_stream_kernel<2, true>>(lds);
      if (err == hipSuccess) hipLaunchKernelGGL((ffn_stream_kernel<2, true>), grid, block, lds, s, a);
    } else {
      err = allow_stream_lds<ffn_stream_kernel<2, false>>(lds);
      if (err == hipSuccess) hipLaunchKernelGGL((ffn_stream_kernel<2, false>), grid, block, lds, s, a);
    }
  }
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace moe
