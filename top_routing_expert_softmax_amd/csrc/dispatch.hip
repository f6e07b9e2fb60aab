// Dispatch: per-expert counting, capacity clip with overflow drop, and the
// stable permutation of (token, choice) pairs into expert-contiguous rows.
// "CMU 11-868 Lecture 17", sections 2.2 (group by expert) and 2.4 (capacity
// and drop).
//
// The rank of pair (t, j) with expert e is #{t' < t : e in S_t'}; a token
// picks each expert at most once, so token order alone fixes it.
//   1. count_rank: each block takes a contiguous token range (blocks of 256
//      threads, one token per thread, chunks of 256 tokens).  Per wavefront
//      and expert an LDS 64-bit mask records which lanes picked the expert;
//      popcount of the lower lanes gives the rank inside the wave, popcounts
//      of earlier waves' masks and the block's running count the rest.
//      The in-block rank goes to row_of_pair (scratch use), the block's
//      per-expert totals to the workspace.
//   2. scan: one wavefront per expert scans the per-block totals (at most 64
//      blocks, one lane each), giving each block its base; then counts,
//      kept = min(count, cap), and offsets = exclusive scan of kept.
//   3. scatter: rank = block base + in-block rank; kept iff rank < cap;
//      writes row_of_pair, token_of_row, drop_mask; rows past R get -1.
//   4. gather: x_perm[r] = x[token_of_row[r]], one wavefront per row.
// Only integer atomics on LDS are used; every output is deterministic.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTPB = kDispatchThreads;         // threads (= tokens) per chunk
constexpr int kWavesPB = kTPB / kWave;

struct PermuteWs {
  int32_t* blk;   // [E][kMaxDispatchBlocks] totals, then bases
};

__global__ __launch_bounds__(kTPB) void count_rank_kernel(
    const int32_t* __restrict__ topk_idx, int32_t* __restrict__ row_of_pair,
    int32_t* __restrict__ blk, int nT, int E, int k, int tokens_per_block) {
  extern __shared__ unsigned long long lds_u64[];
  unsigned long long* mask = lds_u64;                                  // [kWavesPB][E]
  int* running = reinterpret_cast<int*>(lds_u64 + kWavesPB * E);       // [E]
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const unsigned long long lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int e = threadIdx.x; e < E; e += kTPB) running[e] = 0;
  const int tb0 = blockIdx.x * tokens_per_block;
  const int tb1 = min(nT, tb0 + tokens_per_block);
  for (int c0 = tb0; c0 < tb1; c0 += kTPB) {
    for (int q = threadIdx.x; q < kWavesPB * E; q += kTPB) mask[q] = 0ull;
    __syncthreads();
    const int t = c0 + threadIdx.x;
    const bool live = t < tb1;
    if (live) {
      for (int j = 0; j < k; ++j) {
        const int e = topk_idx[static_cast<int64_t>(t) * k + j];
        if (e >= 0 && e < E) atomicOr(&mask[wave * E + e], 1ull << lane);
      }
    }
    __syncthreads();
    if (live) {
      for (int j = 0; j < k; ++j) {
        const int e = topk_idx[static_cast<int64_t>(t) * k + j];
        int r = -1;
        if (e >= 0 && e < E) {
          r = running[e] + __popcll(mask[wave * E + e] & lower);
          for (int w = 0; w < wave; ++w) r += __popcll(mask[w * E + e]);
        }
        row_of_pair[static_cast<int64_t>(t) * k + j] = r;
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kTPB) {
      int s = 0;
      for (int w = 0; w < kWavesPB; ++w) s += __popcll(mask[w * E + e]);
      running[e] += s;
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < E; e += kTPB)
    blk[e * kMaxDispatchBlocks + blockIdx.x] = running[e];
}

__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ blk,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int nblk, int E, int cap) {
  __shared__ int kept[256];
  __shared__ int wave_tot[16];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  constexpr int kWavesScan = 16;                 // 1024 threads
  constexpr int kPerWave = 256 / kWavesScan;     // experts per wave, E <= 256
  // every load of the wave first, then the scans
  int vals[kPerWave];
#pragma unroll
  for (int q = 0; q < kPerWave; ++q) {
    const int e = wave + q * kWavesScan;
    vals[q] = (e < E && lane < nblk) ? blk[e * kMaxDispatchBlocks + lane] : 0;
  }
#pragma unroll
  for (int q = 0; q < kPerWave; ++q) {
    const int e = wave + q * kWavesScan;
    if (e >= E) break;
    const int v = vals[q];
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int n = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += n;
    }
    if (lane < nblk) blk[e * kMaxDispatchBlocks + lane] = incl - v;   // block base
    const int total = __shfl(incl, kWave - 1, kWave);
    if (lane == 0) {
      counts[e] = total;
      kept[e] = min(total, cap);
    }
  }
  __syncthreads();
  // offsets = exclusive scan of kept over E <= 256 experts: 4 per thread of
  // the first 64 threads.
  if (wave == 0) {
    int loc[4];
    int s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      loc[q] = (e < E) ? kept[e] : 0;
      s += loc[q];
    }
    int incl = s;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int n = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += n;
    }
    int run = incl - s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < E) offsets[e] = run;
      run += loc[q];
    }
    if (lane == kWave - 1) offsets[E] = incl;
  }
  (void)wave_tot;
}

__global__ __launch_bounds__(kTPB) void scatter_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ blk,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ row_of_pair,
    int32_t* __restrict__ token_of_row, uint8_t* __restrict__ drop_mask, int nT, int E,
    int k, int cap, int tokens_per_block) {
  const int tb0 = blockIdx.x * tokens_per_block;
  const int tb1 = min(nT, tb0 + tokens_per_block);
  for (int t = tb0 + threadIdx.x; t < tb1; t += kTPB) {
    for (int j = 0; j < k; ++j) {
      const int64_t p = static_cast<int64_t>(t) * k + j;
      const int e = topk_idx[p];
      const int r_in = row_of_pair[p];
      int row = -1;
      if (e >= 0 && e < E && r_in >= 0) {
        const int rank = blk[e * kMaxDispatchBlocks + blockIdx.x] + r_in;
        if (rank < cap) {
          row = offsets[e] + rank;
          token_of_row[row] = t;
        }
      }
      row_of_pair[p] = row;
      drop_mask[p] = row < 0 ? 1 : 0;
    }
  }
  // rows past R hold no token
  const int R = offsets[E];
  const int64_t total = static_cast<int64_t>(nT) * k;
  for (int64_t r = R + static_cast<int64_t>(blockIdx.x) * kTPB + threadIdx.x; r < total;
       r += static_cast<int64_t>(gridDim.x) * kTPB)
    token_of_row[r] = -1;
}

// x_perm[r] = x[token_of_row[r]] for r < R: one wavefront per row, 16-byte
// chunks.
__global__ __launch_bounds__(256) void gather_rows_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ token_of_row,
    const int32_t* __restrict__ offsets, uint4* __restrict__ x_perm, int E,
    int row_chunks, int64_t nrows_max) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (r >= nrows_max || r >= offsets[E]) return;
  const int t = token_of_row[r];
  const uint4* src = x + static_cast<int64_t>(t) * row_chunks;
  uint4* dst = x_perm + r * row_chunks;
  for (int c = lane; c < row_chunks; c += kWave) dst[c] = src[c];
}

int dispatch_blocks(int64_t T, int* tokens_per_block) {
  int64_t tpb = kTPB;
  while ((T + tpb - 1) / tpb > kMaxDispatchBlocks) tpb += kTPB;
  *tokens_per_block = static_cast<int>(tpb);
  return static_cast<int>((T + tpb - 1) / tpb);
}

}  // namespace

size_t permute_workspace_bytes(int64_t /*T*/, int E) {
  return static_cast<size_t>(E) * kMaxDispatchBlocks * sizeof(int32_t);
}

hipError_t launch_permute(int64_t T, int64_t d, int E, int k, int64_t cap, bool bf16,
                          const int32_t* topk_idx, const void* x, int32_t* counts,
                          int32_t* offsets, int32_t* token_of_row, int32_t* row_of_pair,
                          uint8_t* drop_mask, void* x_perm, void* ws, hipStream_t s) {
  int tpb = 0;
  const int nblk = dispatch_blocks(T, &tpb);
  int32_t* blk = static_cast<int32_t*>(ws);
  const size_t lds1 = static_cast<size_t>(kWavesPB) * E * 8 + static_cast<size_t>(E) * 4;
  hipLaunchKernelGGL(count_rank_kernel, dim3(nblk), dim3(kTPB), lds1, s, topk_idx,
                     row_of_pair, blk, static_cast<int>(T), E, k, tpb);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, blk, counts, offsets, nblk, E,
                     static_cast<int>(cap));
  hipLaunchKernelGGL(scatter_kernel, dim3(nblk), dim3(kTPB), 0, s, topk_idx, blk, offsets,
                     row_of_pair, token_of_row, drop_mask, static_cast<int>(T), E, k,
                     static_cast<int>(cap), tpb);
  const int elem = bf16 ? 2 : 4;
  const int row_chunks = static_cast<int>(d * elem / 16);
  const int64_t rows = T * k;
  const int rows_per_block = 4;
  const int64_t gblocks = (rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>(gblocks)),
                     dim3(rows_per_block * kWave), 0, s, static_cast<const uint4*>(x),
                     token_of_row, offsets, static_cast<uint4*>(x_perm), E, row_chunks, rows);
  return hipGetLastError();
}

}  // namespace moe
