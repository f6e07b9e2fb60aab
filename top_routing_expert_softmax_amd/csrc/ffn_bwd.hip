// Helpers of the expert-FFN backward pass (bf16): segment offsets, the
// K-major copies of the activations for the weight-gradient GEMMs, and the
// SwiGLU step (which writes its outputs' K-major copies itself).
//
// For one expert with rows X (the gathered tokens), A = X W1^T, B = X W3^T,
// H = SiLU(A) (*) B, O = H W2^T, and output gradient dO:
//   dH = dO W2,  dA = dH (*) B (*) SiLU'(A),  dB = dH (*) SiLU(A)
//   dX = dA W1 + dB W3 = [dA dB] [W1; W3]
//   dW1 = dA^T X,  dW3 = dB^T X,  dW2 = dO^T H
// (the chain rule of the SwiGLU expert, "CMU 11-868 Lecture 17" section
// 5.2).  Rows are "H-indexed": routed rows 0 .. R-1 as in x_perm, shared
// expert s's rows at T*k + s*T.
#include <math.h>

#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTile = 64;   // transpose tile (64 x 64 bf16)

// One wavefront: for segment s (routed e < E, then shared), its first
// H-indexed row, its row count and its column offset in the K-major copies
// (a prefix sum of the counts rounded up to 64).
__global__ __launch_bounds__(kWave) void seg_info_kernel(const int32_t* __restrict__ offsets,
                                                        int* __restrict__ poff,
                                                        int* __restrict__ hstart,
                                                        int* __restrict__ nrows, int E, int Es,
                                                        int T, int k) {
  const int lane = threadIdx.x;
  const int nseg = E + Es;
  constexpr int kPer = 5;                        // nseg <= 272 < 64 * 5
  int pad[kPer];
  int tot = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int s = lane * kPer + q;
    int n = 0, h = 0;
    if (s < E) {
      h = offsets[s];
      n = offsets[s + 1] - h;
    } else if (s < nseg) {
      h = T * k + (s - E) * T;
      n = T;
    }
    if (s < nseg) {
      hstart[s] = h;
      nrows[s] = n;
    }
    pad[q] = (n + 63) / 64 * 64;
    tot += pad[q];
  }
  int incl = tot;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int n = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += n;
  }
  int base = incl - tot;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int s = lane * kPer + q;
    if (s < nseg) poff[s] = base;
    base += pad[q];
  }
  if (lane == kWave - 1) poff[nseg] = incl;
}

// 64 x 64 bf16 tile transpose through LDS, 256 threads.  Loads: 512
// 16-byte chunks (row r, chunk cc), two per thread, stored with the chunk
// index XOR-ed by r/8 so that the column reads below hit 64 distinct banks.
// Then thread (rb = tid % 8, cp = tid / 8) reads the dwords (columns 2cp,
// 2cp+1) of rows 8rb .. 8rb+7 and writes 16 bytes (8 rows) of output rows
// 2cp and 2cp+1; eight consecutive lanes fill one 128-byte output run.
struct TileT {
  uint32_t w[kTile][kTile / 2];
};

__device__ __forceinline__ void tile_store_chunk(TileT& t, int r, int cc, const u32x4_t v) {
  const int p = (cc ^ (r >> 3)) * 4;
  *reinterpret_cast<u32x4_t*>(&t.w[r][p]) = v;
}

// The two output chunks of thread tid: rows 2cp and 2cp+1 of the
// transposed tile, columns 8rb .. 8rb+7.
__device__ __forceinline__ void tile_read_pair(const TileT& t, int tid, u32x4_t& o0, u32x4_t& o1) {
  const int rb = tid & 7, cp = tid >> 3;
  const int flip = (cp >> 2) & 1;               // half of the lanes start on odd rows
  uint32_t D[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int qq = q ^ flip;
    const int r = rb * 8 + qq;
    D[qq] = t.w[r][cp ^ (rb * 4)];
  }
  uint32_t a[4], b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = (D[2 * j] & 0xFFFFu) | (D[2 * j + 1] << 16);
    b[j] = (D[2 * j] >> 16) | (D[2 * j + 1] & 0xFFFF0000u);
  }
  o0 = u32x4_t{a[0], a[1], a[2], a[3]};
  o1 = u32x4_t{b[0], b[1], b[2], b[3]};
}

// K-major copy of H-indexed activations: dst[c][poff[s] + j] = row
// hstart[s] + j of the source (column c), for j < nrows[s], and 0 up to the
// next multiple of 64.  Routed rows come from src; shared rows from
// src_shared[(row - T*k) mod T] when given (x), else from src (H-indexed).
// C is a multiple of 64.
__global__ __launch_bounds__(256) void transpose_seg_kernel(
    const uint16_t* __restrict__ src, const uint16_t* __restrict__ src_shared,
    uint16_t* __restrict__ dst, const int* __restrict__ poff, const int* __restrict__ hstart,
    const int* __restrict__ nrows, int C, int64_t ld, int E, int T, int k) {
  __shared__ TileT tile;
  const int s = blockIdx.z;
  const int n = nrows[s];
  const int npad = poff[s + 1] - poff[s];
  const int j0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  if (j0 >= npad) return;
  const int h = hstart[s];
  const int tid = threadIdx.x;
  u32x4_t v[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = tid + 256 * it, j = j0 + (idx >> 3), cc = idx & 7;
    v[it] = u32x4_t{0u, 0u, 0u, 0u};
    if (j < n) {
      const int row = h + j;
      const uint16_t* S = (s >= E && src_shared != nullptr)
          ? src_shared + static_cast<int64_t>((row - T * k) % T) * C
          : src + static_cast<int64_t>(row) * C;
      v[it] = *reinterpret_cast<const u32x4_t*>(S + c0 + cc * 8);
    }
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = tid + 256 * it;
    tile_store_chunk(tile, idx >> 3, idx & 7, v[it]);
  }
  __syncthreads();
  u32x4_t o0, o1;
  tile_read_pair(tile, tid, o0, o1);
  const int rb = tid & 7, c = c0 + 2 * (tid >> 3);
  uint16_t* out = dst + static_cast<int64_t>(c) * ld + poff[s] + j0 + rb * 8;
  *reinterpret_cast<u32x4_t*>(out) = o0;
  *reinterpret_cast<u32x4_t*>(out + ld) = o1;
}

// The SwiGLU step fused with the K-major copies its outputs feed: per 64 x
// 64 tile of segment s (rows j0.., columns c0.. of F), from A, B (ab [2F])
// and dH (dh [F]) it forms dA, dB and H = SiLU(A) (*) B, writes dA and dB
// row-major into g13 (the dX GEMM reads them so) and dA^T, dB^T, H^T
// K-major into dabt [2F][ld] and ht [F][ld] at column poff[s] + j (the
// weight gradients read them so).  Rows past the segment load as zero and
// so give the zero padding up to the next multiple of 64.  H is not kept
// row-major: only its K-major copy is read later.  ab may be g13 itself
// (every element is read before it is written, by the same thread).
__global__ __launch_bounds__(256) void swiglu_bwd_t_kernel(
    const uint16_t* ab, uint16_t* g13, const uint16_t* __restrict__ dh,
    uint16_t* __restrict__ dabt, uint16_t* __restrict__ ht, const int* __restrict__ poff,
    const int* __restrict__ hstart, const int* __restrict__ nrows, int F, int64_t ld) {
  __shared__ TileT tiles[3];                    // dA, dB, H
  const int s = blockIdx.z;
  const int n = nrows[s];
  const int npad = poff[s + 1] - poff[s];
  const int j0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  if (j0 >= npad) return;
  const int h = hstart[s];
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = tid + 256 * it, r = idx >> 3, cc = idx & 7, j = j0 + r;
    u32x4_t qa{0u, 0u, 0u, 0u}, qb = qa, qd = qa;
    const int64_t row = static_cast<int64_t>(h) + j;
    if (j < n) {
      qa = *reinterpret_cast<const u32x4_t*>(ab + row * 2 * F + c0 + cc * 8);
      qb = *reinterpret_cast<const u32x4_t*>(ab + row * 2 * F + F + c0 + cc * 8);
      qd = *reinterpret_cast<const u32x4_t*>(dh + row * F + c0 + cc * 8);
    }
    u32x4_t oa, ob, oh;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t pa = 0u, pb = 0u, ph = 0u;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float a = half ? bf16hi(qa[w]) : bf16lo(qa[w]);
        const float b = half ? bf16hi(qb[w]) : bf16lo(qb[w]);
        const float d = half ? bf16hi(qd[w]) : bf16lo(qd[w]);
        const float sg = 1.0f / (1.0f + __expf(-a));
        const float si = a * sg;
        const uint32_t ga = f32_to_bf16(d * b * sg * (1.0f + a * (1.0f - sg)));
        const uint32_t gb = f32_to_bf16(d * si);
        const uint32_t hh = f32_to_bf16(si * b);
        pa |= ga << (16 * half);
        pb |= gb << (16 * half);
        ph |= hh << (16 * half);
      }
      oa[w] = pa; ob[w] = pb; oh[w] = ph;
    }
    if (j < n) {
      *reinterpret_cast<u32x4_t*>(g13 + row * 2 * F + c0 + cc * 8) = oa;
      *reinterpret_cast<u32x4_t*>(g13 + row * 2 * F + F + c0 + cc * 8) = ob;
    }
    tile_store_chunk(tiles[0], r, cc, oa);
    tile_store_chunk(tiles[1], r, cc, ob);
    tile_store_chunk(tiles[2], r, cc, oh);
  }
  __syncthreads();
  const int rb = tid & 7, c = c0 + 2 * (tid >> 3);
  const int64_t col = poff[s] + j0 + rb * 8;
  u32x4_t o0, o1;
  tile_read_pair(tiles[0], tid, o0, o1);
  *reinterpret_cast<u32x4_t*>(dabt + static_cast<int64_t>(c) * ld + col) = o0;
  *reinterpret_cast<u32x4_t*>(dabt + static_cast<int64_t>(c + 1) * ld + col) = o1;
  tile_read_pair(tiles[1], tid, o0, o1);
  *reinterpret_cast<u32x4_t*>(dabt + static_cast<int64_t>(F + c) * ld + col) = o0;
  *reinterpret_cast<u32x4_t*>(dabt + static_cast<int64_t>(F + c + 1) * ld + col) = o1;
  tile_read_pair(tiles[2], tid, o0, o1);
  *reinterpret_cast<u32x4_t*>(ht + static_cast<int64_t>(c) * ld + col) = o0;
  *reinterpret_cast<u32x4_t*>(ht + static_cast<int64_t>(c + 1) * ld + col) = o1;
}

}  // namespace

hipError_t launch_seg_info(const int32_t* offsets, int* poff, int* hstart, int* nrows, int E,
                           int Es, int64_t T, int k, hipStream_t s) {
  hipLaunchKernelGGL(seg_info_kernel, dim3(1), dim3(kWave), 0, s, offsets, poff, hstart, nrows,
                     E, Es, static_cast<int>(T), k);
  return hipGetLastError();
}

hipError_t launch_transpose_seg(const void* src, const void* src_shared, void* dst,
                                const int* poff, const int* hstart, const int* nrows, int C,
                                int64_t ld, int E, int Es, int64_t T, int k, hipStream_t s) {
  // a segment has at most T rows
  const dim3 grid(static_cast<unsigned>((C + kTile - 1) / kTile),
                  static_cast<unsigned>((T + kTile - 1) / kTile + 1),
                  static_cast<unsigned>(E + Es));
  hipLaunchKernelGGL(transpose_seg_kernel, grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(src), static_cast<const uint16_t*>(src_shared),
                     static_cast<uint16_t*>(dst), poff, hstart, nrows, C, ld, E,
                     static_cast<int>(T), k);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd_t(const void* ab, void* g13, const void* dh, void* dabt, void* ht,
                               const int* poff, const int* hstart, const int* nrows, int E,
                               int Es, int64_t T, int64_t F, int64_t ld, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(F / kTile),
                  static_cast<unsigned>((T + kTile - 1) / kTile + 1),
                  static_cast<unsigned>(E + Es));
  hipLaunchKernelGGL(swiglu_bwd_t_kernel, grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(ab), static_cast<uint16_t*>(g13),
                     static_cast<const uint16_t*>(dh), static_cast<uint16_t*>(dabt),
                     static_cast<uint16_t*>(ht), poff, hstart, nrows, static_cast<int>(F), ld);
  return hipGetLastError();
}

}  // namespace moe
