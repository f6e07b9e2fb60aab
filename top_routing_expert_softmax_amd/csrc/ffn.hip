// Grouped expert FFN over ragged expert segments: "CMU 11-868 Lecture 17"
// section 2.2 (one product per expert on its gathered rows) and section 5.2
// (SwiGLU expert: (SiLU(x W1) (*) x W3) W2), plus the always-on shared
// experts of "MoE routing math" section 2.2, which run as full-T segments.
//
// Segments: routed expert e owns rows offsets[e] .. offsets[e+1] of x_perm
// (and of H and y_perm); shared expert s owns rows 0..T-1 of x, rows
// T*k + s*T + m of H and rows s*T + m of y_shared.  A one-block prep kernel
// cuts every segment into BM-row tiles on the device (no host sync: grids
// are sized for the worst case and idle blocks exit).
//
// Phase 1: H = SiLU(A W1^T) (*) (A W3^T), both products of one column tile
//          in the same block so the gate epilogue is fused; H rounded to
//          the layer dtype.
// Phase 2: Y = H W2^T.
// Both operands are K-contiguous in memory ([rows][K] activations and
// [out][in] weights), which is the layout bf16 MFMA operands want.
//
// bf16, large segments: 256 x 256 output tiles, K slices of 64 streamed
// into LDS by direct-to-LDS loads, v_mfma_f32_32x32x16_bf16 with fp32
// accumulators; four wavefronts of 128 x 128 with the barrier in the middle
// of each slice (gemm_mainloop_p5 on a ring of five operand parts, and
// gemm_mainloop_mid_bmn on a ring of two slices for the MN-contiguous
// backward form).  Tiles of the last,
// partial wave of the chip are split along K and summed in a fixed order
// (gemm_big_kernel).  bf16, decode-sized segments: 128-row tiles with
// register prefetch (gemm_bf16_kernel).  fp32 (small configs): VALU tiles,
// the correctness path.
#include <math.h>

#include <atomic>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = 128;        // rows per tile (bf16 path)
constexpr int kBMf = 64;        // rows per tile (fp32 path)
constexpr int kBK = 64;
constexpr int kLdsStride = kBK + 8;   // bf16 elements per LDS row
constexpr int kThreads = 256;

// Split-K of the last, partial wave of BM x 256 tiles (see gemm_big_kernel):
// at most kMaxSplit parts per tile, each at least kMinSplitSlices K slices,
// and at most kMaxCUs partial tiles in flight.
constexpr int kMaxSplit = 4;
constexpr int kMinSplitSlices = 16;
constexpr int kMaxCUs = 256;

struct FfnArgs {
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
  const int4* tiles;     // (segment, A row, rows, H row)
  const int* ntiles;
  float* sk_partial;     // split-K partial tiles of the last wave (fp32)
  unsigned* sk_count;    // arrivals per split tile: [2][kMaxCUs], phase 1 then 2
  int T, d, E, Es, k, F;
  void* ab;              // PHASE 4: the pre-activations (A, B) as [rows, 2F]
  int ksplit;            // PHASE 5: B rows k < ksplit come from w2 / ws2, the
                         // rest from w3 / ws3 (row k - ksplit)
};

// ---------------------------------------------------------------- tiling --
//
// A tile is (segment, first A row, rows, first H row).  Its x field also
// carries the tile's row group: the large-tile kernel runs the row tiles of
// one group against every column tile before the next group, so the blocks
// an XCD holds at once share weight and activation tiles in its L2.  Groups
// never cross a segment (an expert's weights are streamed once per group)
// and hold at most kTileGroup row tiles: x = segment | size << 16 |
// (index in the group) << 20.
constexpr int kTileGroup = 8;
__device__ __forceinline__ int tile_seg(int x) { return x & 0xFFFF; }
__device__ __forceinline__ int tile_gsize(int x) { return (x >> 16) & 15; }
__device__ __forceinline__ int tile_goff(int x) { return (x >> 20) & 15; }

constexpr int kTableThreads = 256;
constexpr int kTableSegs = 5 * kWave;     // E + Es <= 272 segments, five per lane of wave 0

__global__ __launch_bounds__(kTableThreads) void tile_table_kernel(
    const int32_t* __restrict__ offsets, int4* __restrict__ tiles, int* __restrict__ ntiles,
    int E, int Es, int T, int k, int BM, unsigned* __restrict__ sk_count) {
  // Wave 0 counts each segment's tiles (five segments a lane) and scans
  // them into the segments' first tile indices; then every thread writes
  // tiles t, t + 256, ..., finding its segment by binary search.  (One
  // lane writing all the tiles of its segments took 10-15 us.)
  __shared__ int s_first[kTableSegs + 1];
  __shared__ int s_row0[kTableSegs], s_row1[kTableSegs];
  const int tid = threadIdx.x;
  // arrival counters of the split tiles start at zero in every call
  if (sk_count != nullptr)
    for (int i = tid; i < 2 * kMaxCUs; i += kTableThreads) sk_count[i] = 0u;
  const int nseg = E + Es;
  if (tid < kWave) {
    const int lane = tid;
    // the lane's segment bounds, loaded together (indices clamped to E, so
    // every load is in bounds and none waits behind a branch)
    int o0[5], o1[5];
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int s = lane * 5 + q;
      o0[q] = offsets[min(s, E)];
      o1[q] = offsets[min(s + 1, E)];
    }
    int cnt[5];
    int tot = 0;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int s = lane * 5 + q;
      int rows = 0;
      if (s < E) rows = o1[q] - o0[q];
      else if (s < nseg) rows = T;
      cnt[q] = (rows + BM - 1) / BM;
      tot += cnt[q];
    }
    int incl = tot;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int n = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += n;
    }
    int base = incl - tot;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int s = lane * 5 + q;
      if (s < nseg) {
        s_first[s] = base;
        s_row0[s] = o0[q];
        s_row1[s] = o1[q];
      }
      base += cnt[q];
    }
    if (lane == kWave - 1) {
      s_first[nseg] = incl;
      *ntiles = incl;
    }
  }
  __syncthreads();
  const int total = s_first[nseg];
  for (int t = tid; t < total; t += kTableThreads) {
    // the segment holding tile t: s_first[s] <= t < s_first[s + 1]
    int lo = 0, hi = nseg;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_first[mid] <= t) lo = mid;
      else hi = mid;
    }
    const int s = lo;
    const int i = t - s_first[s];
    const int cnt = s_first[s + 1] - s_first[s];
    // the segment's tiles form ng groups of at most kTileGroup, sizes as
    // even as possible (the first rem groups one larger)
    const int ng = (cnt + kTileGroup - 1) / kTileGroup;
    const int gs = cnt / ng, rem = cnt % ng;
    const int big = rem * (gs + 1);
    int g_first, g_size;
    if (i < big) {
      g_size = gs + 1;
      g_first = i / g_size * g_size;
    } else {
      g_size = gs;
      g_first = big + (i - big) / gs * gs;
    }
    int4 tl;
    tl.x = s | (g_size << 16) | ((i - g_first) << 20);
    if (s < E) {
      const int r0 = s_row0[s] + i * BM;
      tl.y = r0;
      tl.z = min(BM, s_row1[s] - r0);
      tl.w = r0;
    } else {
      const int m0 = i * BM;
      tl.y = m0;
      tl.z = min(BM, T - m0);
      tl.w = T * k + (s - E) * T + m0;
    }
    tiles[t] = tl;
  }
}

// ------------------------------------------------------------- bf16 MFMA --

// SiLU(g) = g * sigmoid(g), with the hardware reciprocal (v_rcp_f32, about
// one ulp) in place of an IEEE division: the value is rounded to bf16
// right after, and the division's ten-instruction sequence made the gate
// epilogue a VALU-bound stretch of every phase-1 tile (the grouped FFN
// 1-2% faster without it).
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

template <int PHASE>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[128 * kLdsStride];

  if (static_cast<int>(blockIdx.x) >= *a.ntiles) return;
  const int4 tl = a.tiles[blockIdx.x];
  const int seg = tile_seg(tl.x), arow0 = tl.y, mrows = tl.z, hrow0 = tl.w;
  const bool routed = seg < a.E;
  const int e = routed ? seg : seg - a.E;
  // segments of at most kStreamMaxRows rows belong to the streaming kernels
  if ((routed ? a.offsets[seg + 1] - a.offsets[seg] : a.T) <= kStreamMaxRows) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave-uniform by construction; readfirstlane lets the compiler keep it
  // (and the buffer resources chosen by it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 1, wn = wave & 1;

  // Problem geometry of this phase.
  const int K = PHASE == 1 ? a.d : a.F;
  const int N = PHASE == 1 ? a.F : a.d;          // output columns
  const int n0 = blockIdx.y * (PHASE == 1 ? 64 : 128);
  const uint16_t* A;
  if (PHASE == 1) {
    A = static_cast<const uint16_t*>(routed ? a.x_perm : a.x) + static_cast<int64_t>(arow0) * K;
  } else {
    A = static_cast<const uint16_t*>(a.H) + static_cast<int64_t>(hrow0) * K;
  }
  const int64_t wstride = static_cast<int64_t>(a.F) * a.d;   // elements per expert matrix

  // Each thread moves 4 A chunks and 4 B chunks of 16 bytes per K step.
  // Rows outside the segment (A) or past N (B) read a clamped, valid row
  // and are zeroed by the mask, so every load is unconditional.
  const int kc = tid & 7;
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  uint32_t valid = 0;     // bit q: A row valid; bit 4+q: B row valid
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = (tid >> 3) + 32 * q;      // tile row 0..127
    const bool av = r < mrows;
    a_src[q] = A + static_cast<int64_t>(av ? r : 0) * K + kc * 8;
    int col;
    const uint16_t* W;
    if (PHASE == 1) {
      col = n0 + (r & 63);
      W = static_cast<const uint16_t*>(r < 64 ? (routed ? a.w1 : a.ws1) : (routed ? a.w3 : a.ws3));
    } else {
      col = n0 + r;
      W = static_cast<const uint16_t*>(routed ? a.w2 : a.ws2);
    }
    const bool bv = col < N;
    b_src[q] = W + e * wstride + static_cast<int64_t>(bv ? col : N - 1) * K + kc * 8;
    valid |= (av ? 1u : 0u) << q;
    valid |= (bv ? 1u : 0u) << (4 + q);
  }

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  u32x4_t ra[4], rb[4];
  const u32x4_t zero = {0u, 0u, 0u, 0u};
#define MOE_LOAD_TILE(k0)                                                          \
  _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                  \
    const u32x4_t va = *reinterpret_cast<const u32x4_t*>(a_src[q] + (k0));        \
    const u32x4_t vb = *reinterpret_cast<const u32x4_t*>(b_src[q] + (k0));        \
    ra[q] = ((valid >> q) & 1u) ? va : zero;                                       \
    rb[q] = ((valid >> (4 + q)) & 1u) ? vb : zero;                                 \
  }

  const int nk = K / kBK;
  MOE_LOAD_TILE(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = (tid >> 3) + 32 * q;
      *reinterpret_cast<u32x4_t*>(&As[r * kLdsStride + kc * 8]) = ra[q];
      *reinterpret_cast<u32x4_t*>(&Bs[r * kLdsStride + kc * 8]) = rb[q];
    }
    __syncthreads();
    if (kt + 1 < nk) { MOE_LOAD_TILE((kt + 1) * kBK); }
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kk = ks * 16 + (lane >> 5) * 8;
      bf16x8_t fa[2], fb[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int r = wm * 64 + mi * 32 + (lane & 31);
        fa[mi] = *reinterpret_cast<const bf16x8_t*>(&As[r * kLdsStride + kk]);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int r = PHASE == 1 ? (ni * 64 + wn * 32 + (lane & 31)) : (wn * 64 + ni * 32 + (lane & 31));
        fb[ni] = *reinterpret_cast<const bf16x8_t*>(&Bs[r * kLdsStride + kk]);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
    }
  }

#undef MOE_LOAD_TILE
  // Epilogue.  32x32 accumulator layout: element v of lane l is row
  // 8*(v/4) + 4*(l/32) + v%4, column l%32.
  if (PHASE == 1) {
    uint16_t* Hout = static_cast<uint16_t*>(a.H) + static_cast<int64_t>(hrow0) * a.F;
    const int col = n0 + wn * 32 + (lane & 31);
    if (col < N) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (row < mrows) {
            const float h = silu_f(acc[mi][0][v]) * acc[mi][1][v];
            Hout[static_cast<int64_t>(row) * a.F + col] = f32_to_bf16(h);
          }
        }
    }
  } else {
    uint16_t* Yout = routed ? static_cast<uint16_t*>(a.y_perm) + static_cast<int64_t>(arow0) * a.d
                            : static_cast<uint16_t*>(a.y_shared) +
                                  static_cast<int64_t>(hrow0 - a.T * a.k) * a.d;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int col = n0 + wn * 64 + ni * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (row < mrows) Yout[static_cast<int64_t>(row) * a.d + col] = f32_to_bf16(acc[mi][ni][v]);
        }
    }
  }
}

// ---------------------------------------------- bf16 MFMA, BM x 256 tiles --
//
// Block tile BM rows x 256 B-rows (BM = kBM2), WAVES wavefronts as WM x
// (WAVES/WM), each owning (BM/WM) x (256*WM/WAVES) outputs in 32 x 32
// blocks of v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  Operand
// tiles move global -> LDS with direct-to-LDS loads (buffer loads for the
// K-contiguous operands; no staging registers) through an NST-stage ring
// of K-slices of BKT elements: while slice s is multiplied, the loads of
// slices s+1 .. s+NST-1 are in flight.  Taller
// tiles carry more rows per weight byte streamed: an expert segment of c
// rows streams its weights ceil(c / BM) times.
// LDS rows hold BKT bf16 (ROW bytes = CH chunks of 16 B).  The LDS has 64
// banks (a 256-byte line holding RPL = 256/ROW rows) and serves a 16-byte
// read 16 lanes at a time; chunk c of row r sits at physical chunk
// c ^ ((r / RPL) % CH), so the fragment reads of 16 consecutive rows touch
// every bank once.  Rows past the segment (A) read as zeros through the
// bounded buffer resource (no memory access; the 64-bit-address loads of
// the MN-contiguous form read a clamped valid row instead), and rows past N
// (B) load a clamped valid row: either way they only feed outputs that the
// epilogue does not store.
//
// Block order: a 1-D grid; each XCD (blocks are dealt to the 8 XCDs round
// robin) takes a contiguous chunk of the live tiles, and inside a chunk
// tiles run by row group (at most kTileGroup row tiles of one segment) x all
// column tiles, column by column, so concurrently resident blocks of one XCD
// share A and B tiles in that XCD's L2, and an expert's weight tiles are
// streamed once for all its row tiles rather than once per group it spans.
constexpr int kBM2 = 256;           // rows per tile, large segments
constexpr int kWM = 2;              // wavefronts along M
constexpr int kBN2 = 256;
constexpr int kXcds = 8;

template <int BKT, int BMT>
struct SliceGeom {
  static constexpr int ROW = BKT * 2;                   // bytes per LDS row
  static constexpr int CH = ROW / 16;                   // 16-byte chunks per row
  static constexpr int RPL = 256 / ROW;                 // rows per 256-byte bank line
  static constexpr int RPI = 1024 / ROW;                // rows per wave DMA instruction
  static constexpr int STAGE = (BMT + kBN2) * ROW;      // bytes per slice
};

// LDS bytes of a ring of NST slices; NST = 5 is the ring of five operand
// parts (half a slice each) of gemm_mainloop_p5
template <int BKT, int BMT, int NST>
constexpr int ring_bytes() {
  return NST == 5 ? 5 * SliceGeom<BKT, BMT>::STAGE / 2 : NST * SliceGeom<BKT, BMT>::STAGE;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt [3:0] and [15:14]; expcnt [6:4] and lgkmcnt
  // [11:8] at their maxima (no wait)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t* lds_row_base) {
  __builtin_amdgcn_global_load_lds(gptr, lds_row_base, 16, 0, 0);
}

// The same 16-byte direct-to-LDS load through a buffer resource: a
// wave-uniform base in scalar registers plus a 32-bit byte offset per lane
// (buffer_load_dwordx4 ... lds).  On the grouped GEMM this measured 4-7%
// faster than the 64-bit-address form.  Offsets stay below 2^31: an
// operand tile spans at most 256 rows of K < 2^22 bf16 values.
// bytes: the resource's extent; loads past it return zeros without a
// memory access (raw buffer range check).
// Callers pass wave-uniform values; reading them from the first lane keeps
// the descriptor in scalar registers (a descriptor the compiler takes for
// divergent costs a loop around every load that uses it).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base,
                                                            int bytes = 0x7FFFFFFF) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, static_cast<short>(0),
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t byte_off,
                                              void* lds_row_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)(lds_row_base), 16,
      byte_off, 0, 0, 0);
}

// K loop of one wave: stream slices of A and B into the LDS ring with DMA
// loads and run the wave's MFMAs on them.  MIA (0..MI) is the number of
// the wave's MI 32-row blocks that hold segment rows; the others take no
// MFMA work.  Every wave of the block runs the same loads and barriers.
// B tile rows of an MN-contiguous operand: BKT rows (k) of kBN2 columns.
constexpr int kBRowMN = kBN2 * 2;                       // bytes per LDS row

// Two LDS transpose reads (4 x 16 bit each) make one 8-value MFMA operand.
// In each group of 16 lanes, lane 4p+m receives in slot q element m of the
// 8 bytes that lane 4q+p addresses; so with lane 4q+p pointing at row
// k0+q, column n0+4p of an MN-contiguous tile, lane i gets column n0+i,
// rows k0..k0+3.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8_t lds_read_tr_pair(const char* p, int second) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + second));
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// BMN: the B operand is MN-contiguous (rows of k in global memory and in
// LDS); slice k0 of B then starts k0 rows further on, and b_jump more
// elements from b_kjump on (a second matrix continues the K range).
// BUF: the K-contiguous operands are read through buffer resources (ra,
// rb) at per-lane byte offsets (aoff, boff) instead of the pointers asrc,
// bsrc; slice k0 adds 2 k0 bytes.
struct BufOperands {
  __amdgpu_buffer_rsrc_t ra, rb;
};

template <int BKT, int BMT, int NST, int NIA, int NIB, int MI, int NB, int MIA, bool BMN,
          bool BUF = false>
__device__ __forceinline__ void gemm_mainloop(
    f32x16_t (&acc)[MI][NB], const uint16_t* const (&asrc)[NIA],
    const uint16_t* const (&bsrc)[NIB], char* lds_bytes, int a_dst, int b_dst,
    const int (&a_off)[MI], const int (&b_off)[NB], int lane, int nk, int64_t b_kstride,
    int b_kjump, int64_t b_jump, const BufOperands& bo = BufOperands{},
    const uint32_t* aoff = nullptr, const uint32_t* boff = nullptr) {
  using G = SliceGeom<BKT, BMT>;
  static_assert(!(BUF && BMN), "buffer loads serve the K-contiguous operands");
#define MOE_BK(k0) (BMN ? static_cast<int64_t>(k0) * b_kstride + ((k0) >= b_kjump ? b_jump : 0) \
                        : static_cast<int64_t>(k0))
#define MOE_ISSUE_SLICE(slot, k0)                                                          \
  _Pragma("unroll") for (int i = 0; i < NIA; ++i) {                                        \
    char* d_ = lds_bytes + (slot) * G::STAGE + a_dst + i * G::RPI * G::ROW;               \
    if constexpr (BUF) lds_dma16_buf(bo.ra, aoff[i] + 2u * static_cast<uint32_t>(k0), d_); \
    else lds_dma16(asrc[i] + (k0), reinterpret_cast<uint32_t*>(d_));                      \
  }                                                                                        \
  _Pragma("unroll") for (int i = 0; i < NIB; ++i) {                                        \
    char* d_ = lds_bytes + (slot) * G::STAGE + b_dst + i * 1024;                           \
    if constexpr (BUF) lds_dma16_buf(bo.rb, boff[i] + 2u * static_cast<uint32_t>(k0), d_); \
    else lds_dma16(bsrc[i] + MOE_BK(k0), reinterpret_cast<uint32_t*>(d_));                 \
  }
  // fragment rows are 32-aligned bases + lane%32, so the swizzle key of
  // all of this lane's fragment rows is ((lane % 32) / RPL) % CH
  const int key = ((lane & 31) / G::RPL) % G::CH;
  const int khalf = lane >> 5;
  // prologue: slices 0 .. NST-2 in flight
#pragma unroll
  for (int s0 = 0; s0 < NST - 1; ++s0)
    if (s0 < nk) { MOE_ISSUE_SLICE(s0, s0 * BKT); }
  for (int kt = 0; kt < nk; ++kt) {
    const int slot = kt % NST;
    // slice kt has landed once at most (NST-2) younger slices are pending
    if (kt + NST - 2 < nk) {
      wait_vmcnt<(NST - 2) * (NIA + NIB)>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();            // every wave's part of slice kt is in LDS, and
                                // slot (kt-1) % NST is no longer read
    // An MN-contiguous B is read with LDS transpose reads, which the
    // compiler does not tell apart from the LDS-DMA writes in flight: it
    // would wait for the next slice's loads before the first of them.  So
    // the whole slice's B fragments are read here, before that DMA issue.
    bf16x8_t fbs[BMN ? BKT / 16 : 1][NB];
    if constexpr (BMN) {
      if (MIA > 0) {
        const char* sb = lds_bytes + slot * G::STAGE;
#pragma unroll
        for (int ks = 0; ks < BKT / 16; ++ks)
#pragma unroll
          for (int ni = 0; ni < NB; ++ni)
            fbs[ks][ni] = lds_read_tr_pair(sb + b_off[ni] + ks * 16 * kBRowMN, 4 * kBRowMN);
      }
    }
    {
      // always issue (one block of code for the scheduler): past the last
      // slice, reload the last slice into the free slot
      const int s_next = kt + NST - 1;
      MOE_ISSUE_SLICE(s_next % NST, min(s_next, nk - 1) * BKT);
    }
    if (MIA == 0) continue;
    const char* sb = lds_bytes + slot * G::STAGE;
    __builtin_amdgcn_s_setprio(1);       // the MFMA issue ahead of other waves' loads
#pragma unroll
    for (int ks = 0; ks < BKT / 16; ++ks) {
      const int pc = ((2 * ks + khalf) ^ key) * 16;
      bf16x8_t fa[MIA > 0 ? MIA : 1], fb[NB];
#pragma unroll
      for (int mi = 0; mi < MIA; ++mi) fa[mi] = *reinterpret_cast<const bf16x8_t*>(sb + a_off[mi] + pc);
#pragma unroll
      for (int ni = 0; ni < NB; ++ni) {
        if constexpr (BMN)
          fb[ni] = fbs[ks][ni];
        else
          fb[ni] = *reinterpret_cast<const bf16x8_t*>(sb + b_off[ni] + pc);
      }
#pragma unroll
      for (int mi = 0; mi < MIA; ++mi)
#pragma unroll
        for (int ni = 0; ni < NB; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
      __builtin_amdgcn_iglp_opt(0);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  wait_vmcnt<0>();              // the extra loads of the last iterations
#undef MOE_ISSUE_SLICE
#undef MOE_BK
}

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// The loop of the four-wave tiles (one wave per SIMD, 128 x 128 outputs
// each, K-contiguous operands through buffer resources), on K slices of 64
// with one barrier in the middle of each slice.  The fragments are read
// one half-slice (two 16-wide K steps) ahead into the other of two
// register sets, so the MFMAs do not wait on the LDS at the barrier:
//   phase A of slice s: the MFMAs of its first half (in registers), the
//     reads of its second half, the DMA of A(s+2);
//   barrier: slice s+1 has landed, and every wave is done reading slice s
//     (its last reads belong to phase A);
//   phase B: the MFMAs of the second half, the reads of slice s+1's first
//     half, the DMA of B(s+2).
// The LDS holds the operands' slice parts (256 rows of A or of B, 32 KB
// each) in a ring of five part slots, all 160 KB: part q of the sequence
// A0 B0 A1 B1 ... sits in slot q % 5.  A(s+2) goes to B(s-1)'s slot (free
// since the previous barrier), B(s+2) to A(s)'s; at the barrier of slice s
// only A(s+2)'s loads may still be in flight.  With a ring of two slices
// (no spare slot) both parts of slice s+2 had to load in phase B, and the
// address unit, busy with them for most of that phase, held up the MFMA
// issue: spreading the DMA over both phases made the grouped GEMM 1-3%
// faster.  The MFMAs, fragment reads and DMA issues are interleaved evenly
// by scheduling groups.
template <int BKT, int BMT, int NIA, int NIB, int MI, int NB, int MIA>
__device__ __forceinline__ void gemm_mainloop_p5(
    f32x16_t (&acc)[MI][NB], char* lds_bytes, int a_dst, int b_dst,
    const int (&a_off)[MI], const int (&b_off)[NB], int lane, int nk, const BufOperands& bo,
    const uint32_t (&aoff)[NIA], const uint32_t (&boff)[NIB]) {
  using G = SliceGeom<BKT, BMT>;
  static_assert(BKT == 64 && BMT == kBN2, "a slice is two halves; A and B parts of equal size");
  constexpr int PART = BMT * G::ROW;                // bytes of one operand's slice part
  constexpr int NSLOT = 5;
  constexpr int NMF = 2 * MIA * NB;                 // MFMAs per half-slice
  constexpr int NRD = MIA > 0 ? 2 * (MIA + NB) : 0; // fragment reads per half-slice
  constexpr int MA = MIA > 0 ? MIA : 1;
  const int key = ((lane & 31) / G::RPL) % G::CH;
  const int khalf = lane >> 5;
  bf16x8_t ra[2][2][MA], rb[2][2][NB];              // [set][k16 step of the half][block]
  // B rows follow the A rows within a slice in the callers' offsets
  const int bd = b_dst - PART;

#define P5_DMA_A(pslot, k0, d)                                                                  \
  lds_dma16_buf(bo.ra, aoff[d] + 2u * static_cast<uint32_t>(k0),                                \
                lds_bytes + (pslot) * PART + a_dst + (d) * G::RPI * G::ROW)
#define P5_DMA_B(pslot, k0, d)                                                                  \
  lds_dma16_buf(bo.rb, boff[d] + 2u * static_cast<uint32_t>(k0),                                \
                lds_bytes + (pslot) * PART + bd + (d) * G::RPI * G::ROW)
#define P5_RD(set, aslot, bslot, h, r)                                                          \
  do {                                                                                          \
    const int j_ = (r) / (MIA + NB), q_ = (r) % (MIA + NB);                                     \
    const int pc_ = ((2 * (2 * (h) + j_) + khalf) ^ key) * 16;                                  \
    if (q_ < MIA)                                                                               \
      ra[set][j_][q_ < MIA ? q_ : 0] = *reinterpret_cast<const bf16x8_t*>(                      \
          lds_bytes + (aslot) * PART + a_off[q_ < MIA ? q_ : 0] + pc_);                         \
    else                                                                                        \
      rb[set][j_][q_ >= MIA ? q_ - MIA : 0] = *reinterpret_cast<const bf16x8_t*>(               \
          lds_bytes + (bslot) * PART - PART + b_off[q_ >= MIA ? q_ - MIA : 0] + pc_);           \
  } while (0)
#define P5_MF(set, m)                                                                           \
  do {                                                                                          \
    const int j_ = (m) / (MIA * NB), t_ = (m) % (MIA * NB);                                     \
    const int mi_ = t_ / NB, ni_ = t_ % NB;                                                     \
    acc[mi_][ni_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[set][j_][mi_], rb[set][j_][ni_], \
                                                            acc[mi_][ni_], 0, 0, 0);            \
  } while (0)
  // one half-slice: the MFMAs of register set SET, the reads of half H of
  // the parts in slots AS, BS into the other set, and NDM DMA issues
#define P5_PHASE(SET, AS, BS, H, NDM, DMA)                                                      \
  do {                                                                                          \
    if constexpr (MIA > 0) {                                                                    \
      _Pragma("unroll") for (int m = 0; m < NMF; ++m) {                                         \
        P5_MF(SET, m);                                                                          \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                      \
        _Pragma("unroll") for (int d = 0; d < (NDM); ++d) {                                     \
          if ((d * NMF) / (NDM) == m) {                                                         \
            DMA(d);                                                                             \
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                  \
          }                                                                                     \
        }                                                                                       \
        _Pragma("unroll") for (int r = 0; r < NRD; ++r) {                                       \
          const int at = ((r + 1) * NMF) / NRD - 1;                                             \
          if ((at < 0 ? 0 : at) == m) {                                                         \
            P5_RD(1 - (SET), AS, BS, H, r);                                                     \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                  \
          }                                                                                     \
        }                                                                                       \
      }                                                                                         \
    } else {                                                                                    \
      _Pragma("unroll") for (int d = 0; d < (NDM); ++d) DMA(d);                                 \
    }                                                                                           \
  } while (0)

  // prologue: A0 B0 A1 B1 in slots 0 .. 3; slice 0 landed and its first
  // half read
  {
    const int k1 = min(1, nk - 1) * BKT;
#pragma unroll
    for (int d = 0; d < NIA; ++d) P5_DMA_A(0, 0, d);
#pragma unroll
    for (int d = 0; d < NIB; ++d) P5_DMA_B(1, 0, d);
#pragma unroll
    for (int d = 0; d < NIA; ++d) P5_DMA_A(2, k1, d);
#pragma unroll
    for (int d = 0; d < NIB; ++d) P5_DMA_B(3, k1, d);
  }
  wait_vmcnt<NIA + NIB>();
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (MIA > 0) {
#pragma unroll
    for (int r = 0; r < NRD; ++r) P5_RD(0, 0, 1, 0, r);
  }
  int qa = 0;                                       // slot of A(s); B(s) in the next
  for (int s = 0; s < nk; ++s) {
    const int qb = qa + 1 < NSLOT ? qa + 1 : qa + 1 - NSLOT;
    const int qna = qa + 2 < NSLOT ? qa + 2 : qa + 2 - NSLOT;
    const int qnb = qa + 3 < NSLOT ? qa + 3 : qa + 3 - NSLOT;
    const int qda = qa + 4 < NSLOT ? qa + 4 : qa + 4 - NSLOT;
    const int k2 = min(s + 2, nk - 1) * BKT;
    // phase A: A(s+2) into B(s-1)'s slot
#define P5_DA(d) P5_DMA_A(qda, k2, d)
    P5_PHASE(0, qa, qb, 1, NIA, P5_DA);
#undef P5_DA
    wait_lgkm0();
    wait_vmcnt<NIA>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // phase B: B(s+2) into A(s)'s slot; slice s+1's first half read
#define P5_DB(d) P5_DMA_B(qa, k2, d)
    P5_PHASE(1, qna, qnb, 0, NIB, P5_DB);
#undef P5_DB
    qa = qna;
  }
  wait_vmcnt<0>();
  wait_lgkm0();
#undef P5_PHASE
#undef P5_DMA_A
#undef P5_DMA_B
#undef P5_RD
#undef P5_MF
}

// The mid-slice-barrier loop for the MN-contiguous form (phase 5, dH and
// dX on the weights as stored), four waves of 128 x 128, on a ring of two
// slices.  Its B fragments come from LDS transpose reads, before which the
// compiler waits for every LDS-DMA load in flight; so a whole slice's B
// fragments are read at the start of phase B, right after the barrier
// (when no load is in flight), into the other of two slice-sized register
// sets, and the DMA of slice s+2 (both operands) follows them in phase B.
// (The five-part ring of gemm_mainloop_p5 would put loads in flight at
// that point.)  Only the A fragments (ordinary reads) are read a
// half-slice ahead as in gemm_mainloop_p5.  Operands through 64-bit
// addresses (asrc, bsrc; B advancing k0 * b_kstride, plus b_jump from
// K = b_kjump on).
template <int BKT, int BMT, int NIA, int NIB, int MI, int NB, int MIA>
__device__ __forceinline__ void gemm_mainloop_mid_bmn(
    f32x16_t (&acc)[MI][NB], const uint16_t* const (&asrc)[NIA],
    const uint16_t* const (&bsrc)[NIB], char* lds_bytes, int a_dst, int b_dst,
    const int (&a_off)[MI], const int (&b_off)[NB], int lane, int nk, int64_t b_kstride,
    int b_kjump, int64_t b_jump) {
  using G = SliceGeom<BKT, BMT>;
  static_assert(BKT == 64, "a slice is two halves of two 16-wide K steps");
  constexpr int NDMA = NIA + NIB;
  constexpr int MA = MIA > 0 ? MIA : 1;
  constexpr int NMF = 2 * MIA * NB;                 // MFMAs per half-slice
  constexpr int NRA = 2 * MIA;                      // A fragment reads per half-slice
  const int key = ((lane & 31) / G::RPL) % G::CH;
  const int khalf = lane >> 5;
  bf16x8_t ra[2][2][MA];                            // [set][k16 step of the half][mi]
  bf16x8_t rb[2][4][NB];                            // [set][k16 step of the slice][ni]
#define MOE_BK(k0) (static_cast<int64_t>(k0) * b_kstride + ((k0) >= b_kjump ? b_jump : 0))
#define MOE_MDMA(slot, k0, d)                                                                   \
  do {                                                                                          \
    if ((d) < NIA)                                                                              \
      lds_dma16(asrc[(d) < NIA ? (d) : 0] + (k0),                                               \
                reinterpret_cast<uint32_t*>(lds_bytes + (slot) * G::STAGE + a_dst +             \
                                            ((d) < NIA ? (d) : 0) * G::RPI * G::ROW));          \
    else                                                                                        \
      lds_dma16(bsrc[(d) >= NIA ? (d) - NIA : 0] + MOE_BK(k0),                                  \
                reinterpret_cast<uint32_t*>(lds_bytes + (slot) * G::STAGE + b_dst +             \
                                            ((d) >= NIA ? (d) - NIA : 0) * 1024));              \
  } while (0)
#define MOE_MRDA(set, slot, h, r)                                                               \
  do {                                                                                          \
    const int j_ = (r) / MA, q_ = (r) % MA;                                                     \
    const int pc_ = ((2 * (2 * (h) + j_) + khalf) ^ key) * 16;                                  \
    ra[set][j_][q_] = *reinterpret_cast<const bf16x8_t*>(lds_bytes + (slot) * G::STAGE +        \
                                                         a_off[q_] + pc_);                      \
  } while (0)
#define MOE_MRDB(set, slot)                                                                     \
  _Pragma("unroll") for (int ks_ = 0; ks_ < 4; ++ks_)                                           \
    _Pragma("unroll") for (int ni_ = 0; ni_ < NB; ++ni_)                                        \
      rb[set][ks_][ni_] = lds_read_tr_pair(lds_bytes + (slot) * G::STAGE + b_off[ni_] +         \
                                           ks_ * 16 * kBRowMN, 4 * kBRowMN)
#define MOE_MMF(aset, bset, h, m)                                                               \
  do {                                                                                          \
    const int j_ = (m) / (MIA * NB), t_ = (m) % (MIA * NB);                                     \
    const int mi_ = t_ / NB, ni_ = t_ % NB;                                                     \
    acc[mi_][ni_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                                    \
        ra[aset][j_][mi_], rb[bset][2 * (h) + j_][ni_], acc[mi_][ni_], 0, 0, 0);                \
  } while (0)

  // prologue: slices 0 and 1 in flight; slice 0 landed, its A first half
  // and all its B fragments read
#pragma unroll
  for (int d = 0; d < NDMA; ++d) MOE_MDMA(0, 0, d);
#pragma unroll
  for (int d = 0; d < NDMA; ++d) MOE_MDMA(1, min(1, nk - 1) * BKT, d);
  wait_vmcnt<0>();
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (MIA > 0) {
#pragma unroll
    for (int r = 0; r < NRA; ++r) MOE_MRDA(0, 0, 0, r);
  }
  MOE_MRDB(0, 0);

  // one iteration on slice S whose B fragments sit in register set BSET
#define MOE_MITER(S, BSET)                                                                      \
  do {                                                                                          \
    const int s_ = (S);                                                                         \
    const int slot_ = s_ & 1;                                                                   \
    if constexpr (MIA > 0) {                                                                    \
      _Pragma("unroll") for (int m = 0; m < NMF; ++m) {                                         \
        MOE_MMF(0, BSET, 0, m);                                                                 \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                      \
        _Pragma("unroll") for (int r = 0; r < NRA; ++r) {                                       \
          if ((((r + 1) * NMF) / NRA - 1) == m) {                                               \
            MOE_MRDA(1, slot_, 1, r);                                                           \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                  \
          }                                                                                     \
        }                                                                                       \
      }                                                                                         \
    }                                                                                           \
    wait_lgkm0();                                                                               \
    wait_vmcnt<0>();                                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    __builtin_amdgcn_s_barrier();                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    /* slice s+1's B fragments, with no load in flight */                                       \
    MOE_MRDB(1 - (BSET), slot_ ^ 1);                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    const int kn_ = min(s_ + 2, nk - 1) * BKT;                                                  \
    if constexpr (MIA > 0) {                                                                    \
      _Pragma("unroll") for (int m = 0; m < NMF; ++m) {                                         \
        MOE_MMF(1, BSET, 1, m);                                                                 \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                      \
        _Pragma("unroll") for (int d = 0; d < NDMA; ++d) {                                      \
          if ((d * NMF) / NDMA == m) {                                                          \
            MOE_MDMA(slot_, kn_, d);                                                            \
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                  \
          }                                                                                     \
        }                                                                                       \
        _Pragma("unroll") for (int r = 0; r < NRA; ++r) {                                       \
          if ((((r + 1) * NMF) / NRA - 1) == m) {                                               \
            MOE_MRDA(0, slot_ ^ 1, 0, r);                                                       \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                  \
          }                                                                                     \
        }                                                                                       \
      }                                                                                         \
    } else {                                                                                    \
      _Pragma("unroll") for (int d = 0; d < NDMA; ++d) MOE_MDMA(slot_, kn_, d);                 \
    }                                                                                           \
  } while (0)
  for (int s = 0; s < nk; s += 2) {
    MOE_MITER(s, 0);
    if (s + 1 < nk) MOE_MITER(s + 1, 1);
  }
  wait_vmcnt<0>();
  wait_lgkm0();
#undef MOE_MITER
#undef MOE_MMF
#undef MOE_MRDB
#undef MOE_MRDA
#undef MOE_MDMA
#undef MOE_BK
}

// ---- epilogue through the LDS.  The block's bf16 output tile (BMT rows x
// COLS columns) is first written into the idle LDS ring, its 16-byte chunks
// XOR-swizzled by row (chunk c of row r at c ^ (r % NCH)), so that the two
// half-waves of a write (rows r and r + 4, 32 columns each) fall in
// different banks; then consecutive threads copy consecutive chunks of a
// row to memory, so every store instruction writes whole 16-byte pieces of
// full rows instead of 2 bytes per lane.
// HW: round with the hardware conversion (the inference phases 1 and 2,
// 0.5-1% faster there), else with integer arithmetic (same bits).
template <int COLS, bool HW>
__device__ __forceinline__ void stage_put(char* lds, int row, int col, float v) {
  constexpr int NCH = COLS / 8;
  const int off = row * (COLS * 2) + (((col >> 3) ^ (row & (NCH - 1))) << 4) + ((col & 7) << 1);
  *reinterpret_cast<uint16_t*>(lds + off) = HW ? f32_to_bf16_hw(v) : f32_to_bf16(v);
}

// dst(row, chunk) gives the destination of 16-byte chunk `chunk` of tile row
// `row`, or nullptr for a chunk past the matrix's columns.
template <int BMT, int COLS, int NTHR, class Dst>
__device__ __forceinline__ void stage_copy_out(const char* lds, int tid, int mrows, Dst dst) {
  constexpr int NCH = COLS / 8;
  static_assert((BMT * NCH) % NTHR == 0, "whole chunks per thread");
#pragma unroll
  for (int j = 0; j < BMT * NCH / NTHR; ++j) {
    const int i = j * NTHR + tid;
    const int row = i / NCH, ch = i % NCH;
    if (row >= mrows) continue;
    uint16_t* p = dst(row, ch);
    if (p == nullptr) continue;
    *reinterpret_cast<u32x4_t*>(p) = *reinterpret_cast<const u32x4_t*>(
        lds + row * (COLS * 2) + ((ch ^ (row & (NCH - 1))) << 4));
  }
}

template <int PHASE, int BKT, int NST, int WAVES, int BMT, int WMW>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4)))
void gemm_big_kernel(FfnArgs a, int NT, int ncu) {
  using G = SliceGeom<BKT, BMT>;
  constexpr int WN = WAVES / WMW;           // waves along N
  constexpr int WR = BMT / WMW;             // output rows per wave
  constexpr int MI = WR / 32;               // 32-row blocks per wave
  constexpr int NB = kBN2 / WN / 32;        // 32-wide B blocks per wave
  constexpr int AROWS = BMT / WAVES;        // A tile rows each wave loads
  constexpr int BROWS = kBN2 / WAVES;       // B tile rows each wave loads
  constexpr int NIA = AROWS / G::RPI;       // DMA instructions per wave, A
  constexpr int NIB = BROWS / G::RPI;       // DMA instructions per wave, B
  static_assert(MI * 32 == WR && MI >= 1 && MI <= 4, "tile rows per wave");
  static_assert(NIA * G::RPI == AROWS && NIB * G::RPI == BROWS, "DMA rows");
  static_assert(NB >= 2 && NB % 2 == 0, "tile columns per wave");
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];

  // ---- which tile, and which part of its K range
  // The L = MT * NT tiles fill L / ncu whole waves of the chip (one block
  // per CU).  A partial last wave of r tiles would leave CUs idle, so
  // those r tiles are split along K into S parts that run as separate
  // blocks; each part writes an fp32 partial tile, and the block that
  // arrives last sums the S partials in part order (so the result does not
  // depend on arrival order) and runs the epilogue.
  const int MT = *a.ntiles;
  const int L = MT * NT;
  // PHASE 3 is phase 1 with the gate and up products stored apart (the
  // recompute of the backward pass); PHASE 4 stores both H and the two
  // products (a forward that keeps what its backward needs)
  // PHASE 5 is the phase-2 form with an MN-contiguous B (the backward's
  // dH = dO W2 and dX = [dA dB] [W1; W3] on the weights as stored)
  constexpr bool P1 = PHASE == 1 || PHASE == 3 || PHASE == 4;
  constexpr bool BMN = PHASE == 5;
  // four waves of 128 x 128 run the mid-slice-barrier loops (NST = 5: the
  // ring of five operand parts)
  constexpr bool kMidBmn = WAVES == 4 && BMN && BKT == 64 && NST == 2;
  constexpr bool kPart5 = WAVES == 4 && !BMN && BKT == 64 && NST == 5;
  const int K = P1 ? a.d : a.F;
  const int nk_all = K / BKT;
  const int r = L % ncu;
  int S = 1;
  if (r > 0) {
    const int rr = (r + kXcds - 1) / kXcds * kXcds;
    S = min(min(kMaxSplit, ncu / rr), nk_all / kMinSplitSlices);
    if (S < 2) S = 1;
  }
  const int D = S > 1 ? L - r : L;              // tiles that run whole
  const int chunk = (D + kXcds - 1) / kXcds;
  const int b = blockIdx.x;
  int pid, part = 0, tile_sk = 0;
  const bool split_unit = b >= kXcds * chunk;
  if (!split_unit) {
    const int xcd = b % kXcds;
    const int j = b / kXcds;
    pid = xcd * chunk + j;
    if (pid >= D) return;
  } else {
    if (S == 1) return;
    // the S parts of a split tile go to blocks of one XCD
    const int u = b - kXcds * chunk;
    tile_sk = u % kXcds + kXcds * (u / (kXcds * S));
    part = (u / kXcds) % S;
    if (tile_sk >= r) return;
    pid = D + tile_sk;
  }
  const int parts = split_unit ? S : 1;         // whole tiles take all of K
  const int kb = part * nk_all / parts;
  const int nk = (part + 1) * nk_all / parts - kb;
  // pid / NT lies in pid's row group, since a group spans every column
  const int mt0 = pid / NT;
  // The row group of mt0 holds at most kTileGroup row tiles, so the tile
  // this block takes lies within kTileGroup - 1 of mt0: one vector load of
  // that window (an entry a lane, clamped to the table) in place of two
  // dependent scalar loads (the group, then the tile): 0.2-0.4% faster.
  const int wlane = threadIdx.x & (kWave - 1);
  const int4 wv = a.tiles[min(max(mt0 - (kTileGroup - 1) + wlane, 0), MT - 1)];
  const int gx = __builtin_amdgcn_readlane(wv.x, kTileGroup - 1);
  const int first_m = mt0 - tile_goff(gx);
  const int gm = tile_gsize(gx);
  const int in_group = pid - first_m * NT;
  const int mt = first_m + in_group % gm;
  const int nt = in_group / gm;
  const int wl = mt - mt0 + (kTileGroup - 1);    // mt's lane of the window
  const int seg = tile_seg(__builtin_amdgcn_readlane(wv.x, wl));
  const int arow0 = __builtin_amdgcn_readlane(wv.y, wl);
  const int mrows = __builtin_amdgcn_readlane(wv.z, wl);
  const int hrow0 = __builtin_amdgcn_readlane(wv.w, wl);
  const bool routed = seg < a.E;
  const int e = routed ? seg : seg - a.E;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave-uniform by construction; readfirstlane lets the compiler keep it
  // (and the buffer resources chosen by it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / WN, wn = wave % WN;

  const int N = P1 ? a.F : a.d;
  const int n0 = nt * (P1 ? kBN2 / 2 : kBN2);
  const uint16_t* A = P1
      ? static_cast<const uint16_t*>(routed ? a.x_perm : a.x) + static_cast<int64_t>(arow0) * K
      : static_cast<const uint16_t*>(a.H) + static_cast<int64_t>(hrow0) * K;
  const int64_t wstride = static_cast<int64_t>(a.F) * a.d;

  // ---- per-lane sources of the DMA instructions of a slice.  Wave w,
  // instruction i covers tile rows w*ROWS + i*RPI .. +RPI of its operand;
  // lane l takes row r = w*ROWS + i*RPI + l/CH and the logical chunk that
  // the swizzle stores at physical chunk l%CH of that row.
  const uint16_t* asrc[NIA];
  const uint16_t* bsrc[NIB];
#pragma unroll
  for (int i = 0; i < NIA; ++i) {
    const int r = wave * AROWS + i * G::RPI + lane / G::CH;
    const int lchunk = (lane % G::CH) ^ ((r / G::RPL) % G::CH);
    const int ra = r < mrows ? r : mrows - 1;
    asrc[i] = A + static_cast<int64_t>(ra) * K + kb * BKT + lchunk * 8;
  }
  int64_t b_kstride = 1, b_jump = 0;
  int b_kjump = 1 << 30;
  if constexpr (BMN) {
    // B tile: BKT rows of kBN2 columns, row k of B = row k of w2 (k <
    // ksplit) or row k - ksplit of w3, each matrix ksplit x N per expert.
    // An instruction covers two rows (32 chunks of 16 bytes each); lane l
    // takes row r = wave * BKT/WAVES + 2i + l/32 and the logical chunk that
    // sits at physical chunk l%32, chunks XOR-ed with 4 (r%4), so the
    // transpose reads of four consecutive rows hit 64 distinct banks.
    static_assert(NIB * 2 == BKT / WAVES, "MN-contiguous B rows per wave");
    const int kabs = kb * BKT;
    const bool second = kabs >= a.ksplit;
    const uint16_t* W2s = static_cast<const uint16_t*>(routed ? a.w2 : a.ws2);
    const uint16_t* W3s = static_cast<const uint16_t*>(routed ? a.w3 : a.ws3);
    const int64_t wst = static_cast<int64_t>(a.ksplit) * N;
    const uint16_t* W = (second ? W3s : W2s) + e * wst;
    const int kbase = second ? kabs - a.ksplit : kabs;
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
      const int r = wave * (BKT / WAVES) + 2 * i + lane / 32;
      const int lchunk = (lane % 32) ^ (4 * (r % 4));
      int col = n0 + lchunk * 8;
      col = col < N ? col : N - 8;
      bsrc[i] = W + static_cast<int64_t>(kbase + r) * N + col;
    }
    b_kstride = N;
    if (!second) {
      b_kjump = a.ksplit - kabs;
      b_jump = (reinterpret_cast<intptr_t>(W3s) - reinterpret_cast<intptr_t>(W2s)) / 2 -
               static_cast<int64_t>(a.ksplit) * N;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
      const int r = wave * BROWS + i * G::RPI + lane / G::CH;
      const int lchunk = (lane % G::CH) ^ ((r / G::RPL) % G::CH);
      int col;
      const uint16_t* W;
      if (P1) {
        col = n0 + (r & 127);
        W = static_cast<const uint16_t*>(r < 128 ? (routed ? a.w1 : a.ws1) : (routed ? a.w3 : a.ws3));
      } else {
        col = n0 + r;
        W = static_cast<const uint16_t*>(routed ? a.w2 : a.ws2);
      }
      col = col < N ? col : N - 1;
      bsrc[i] = W + e * wstride + static_cast<int64_t>(col) * K + kb * BKT + lchunk * 8;
    }
  }
  // The buffer-resource form of the K-contiguous operands: the A tile from
  // its first row, the B tile from column n0 of the wave's matrix (a wave's
  // B rows all lie in W1 or all in W3: 128 is a multiple of BROWS).
  BufOperands bo{};
  uint32_t aoff[NIA], boff[NIB];
  if constexpr (!BMN) {
    // A rows past the segment fall outside the resource and read as zeros
    // without touching memory, so a tail tile streams only its own rows
    // (their products are never stored)
    bo.ra = buffer_rsrc(A, mrows * K * 2);
    const bool w3rows = P1 && wave * BROWS >= 128;
    const uint16_t* Wb = static_cast<const uint16_t*>(
        P1 ? (w3rows ? (routed ? a.w3 : a.ws3) : (routed ? a.w1 : a.ws1))
           : (routed ? a.w2 : a.ws2));
    const uint16_t* Bbase = Wb + e * wstride + static_cast<int64_t>(n0) * K;
    bo.rb = buffer_rsrc(Bbase);
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
      const int r = wave * AROWS + i * G::RPI + lane / G::CH;
      const int lchunk = (lane % G::CH) ^ ((r / G::RPL) % G::CH);
      aoff[i] = static_cast<uint32_t>((static_cast<int64_t>(r) * K + kb * BKT + lchunk * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < NIB; ++i) boff[i] = static_cast<uint32_t>((bsrc[i] - Bbase) * 2);
  }
  char* lds_bytes = reinterpret_cast<char*>(lds);
  const int a_dst = wave * AROWS * G::ROW;
  const int b_dst = BMT * G::ROW + wave * BROWS * G::ROW;

  f32x16_t acc[MI][NB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int jn = 0; jn < NB; ++jn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jn][v] = 0.f;

  // Phase 1: the wave's first NB/2 B blocks are gate (W1) columns, the last
  // NB/2 the same columns of W3.
  int a_off[MI], b_off[NB];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) a_off[mi] = (wm * WR + mi * 32 + (lane & 31)) * G::ROW;
#pragma unroll
  for (int ni = 0; ni < NB; ++ni) {
    if constexpr (BMN) {
      // transpose-read pointers: lane 16g + 4q + p addresses row
      // 8 (g/2) + q, column nb + 16 (g%2) + 4p of the slice
      const int g = lane / 16, q = (lane % 16) / 4, pp = lane % 4;
      const int ncol = wn * (kBN2 / WN) + ni * 32 + 16 * (g % 2) + 4 * pp;
      const int krow = 8 * (g / 2) + q;
      b_off[ni] = BMT * G::ROW + krow * kBRowMN + (((ncol / 8) ^ (4 * q)) * 16) + (ncol % 8) * 2;
    } else {
      const int r = P1
          ? ((ni / (NB / 2)) * 128 + wn * (128 / WN) + (ni % (NB / 2)) * 32 + (lane & 31))
          : (wn * (kBN2 / WN) + ni * 32 + (lane & 31));
      b_off[ni] = BMT * G::ROW + r * G::ROW;
    }
  }

  // 32-row blocks of this wave's WR rows that hold segment rows: a tail
  // tile runs MFMAs only for those.
  const int rows_w = mrows - wm * WR;
  const int mia = __builtin_amdgcn_readfirstlane(
      rows_w <= 0 ? 0 : (rows_w >= WR ? MI : (rows_w + 31) / 32));
#define MOE_MAINLOOP(X)                                                                    \
  {                                                                                         \
  if constexpr (kPart5) {                                                            \
    gemm_mainloop_p5<BKT, BMT, NIA, NIB, MI, NB, (X)>(acc, lds_bytes, a_dst, b_dst, a_off,   \
                                                      b_off, lane, nk, bo, aoff, boff);      \
  } else if constexpr (kMidBmn) {                                                           \
    gemm_mainloop_mid_bmn<BKT, BMT, NIA, NIB, MI, NB, (X)>(acc, asrc, bsrc, lds_bytes, a_dst, \
                                                           b_dst, a_off, b_off, lane, nk,    \
                                                           b_kstride, b_kjump, b_jump);      \
  } else {                                                                                  \
    gemm_mainloop<BKT, BMT, NST, NIA, NIB, MI, NB, (X), BMN, !BMN>(                         \
        acc, asrc, bsrc, lds_bytes, a_dst, b_dst, a_off, b_off, lane, nk, b_kstride,         \
        b_kjump, b_jump, bo, aoff, boff);                                                   \
  }                                                                                         \
  }
  switch (mia) {
    case 4: if constexpr (MI >= 4) MOE_MAINLOOP(MI >= 4 ? 4 : 0); break;
    case 3: if constexpr (MI >= 3) MOE_MAINLOOP(MI >= 3 ? 3 : 0); break;
    case 2: if constexpr (MI >= 2) MOE_MAINLOOP(MI >= 2 ? 2 : 0); break;
    case 1: MOE_MAINLOOP(1); break;
    default: MOE_MAINLOOP(0); break;
  }
#undef MOE_MAINLOOP

  if (split_unit) {
    // Partial tile in accumulator order: float4 q of accumulator (mi, ni)
    // of thread tid sits at ((mi * NB + ni) * 4 + q) * NTHR + tid.
    constexpr int NTHR = WAVES * kWave;
    constexpr int64_t kSlot = static_cast<int64_t>(BMT) * kBN2 / 4;   // float4 per tile
    f32x4_t* mine = reinterpret_cast<f32x4_t*>(a.sk_partial) +
                    static_cast<int64_t>(tile_sk * S + part) * kSlot;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NB; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4_t v = {acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                       acc[mi][ni][4 * q + 3]};
          mine[((mi * NB + ni) * 4 + q) * NTHR + tid] = v;
        }
    // Release the partial device-wide, then count the arrival; the last of
    // the S parts takes the tile.  The LDS ring is idle by now (every wave
    // is past its K loop), so its first word carries the verdict.
    __threadfence();
    __syncthreads();
    int* flag = reinterpret_cast<int*>(lds_bytes);
    unsigned* count = &a.sk_count[(P1 ? 0 : kMaxCUs) + tile_sk];
    if (tid == 0) {
      const bool last = atomicAdd(count, 1u) == static_cast<unsigned>(S - 1);
      // the last part leaves the counter at zero for the next launch
      if (last) *count = 0u;
      *flag = last;
    }
    __syncthreads();
    if (*flag == 0) return;
    __threadfence();            // acquire: the other parts' partials
    const f32x4_t* first = reinterpret_cast<const f32x4_t*>(a.sk_partial) +
                           static_cast<int64_t>(tile_sk * S) * kSlot;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NB; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t at = ((mi * NB + ni) * 4 + q) * NTHR + tid;
          f32x4_t v = first[at];
          for (int p = 1; p < S; ++p) v += first[static_cast<int64_t>(p) * kSlot + at];
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[mi][ni][4 * q + c] = v[c];
        }
  }

  // ---- epilogue (accumulator element v of lane l: row 8*(v/4) + 4*(l/32)
  // + v%4, column l%32 of its 32 x 32 block), staged through the LDS ring,
  // idle once every wave is past its K loop.
  constexpr int NTHR = WAVES * kWave;
  static_assert(BMT * 256 * 2 <= ring_bytes<BKT, BMT, NST>(), "the staged tile fits the LDS ring");
  char* stg = lds_bytes;
  if constexpr (PHASE == 1 || PHASE == 4) {
    // H = SiLU(gate) * up: 128 columns from n0 of a [rows, F] matrix
    uint16_t* Hout = static_cast<uint16_t*>(a.H) + static_cast<int64_t>(hrow0) * a.F;
    __syncthreads();
#pragma unroll
    for (int ni = 0; ni < NB / 2; ++ni)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * WR + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const int col = wn * (128 / WN) + ni * 32 + (lane & 31);
          stage_put<128, PHASE == 1>(stg, row, col, silu_f(acc[mi][ni][v]) * acc[mi][ni + NB / 2][v]);
        }
    __syncthreads();
    const int F = a.F;
    stage_copy_out<BMT, 128, NTHR>(stg, tid, mrows, [&](int row, int ch) -> uint16_t* {
      const int col = n0 + ch * 8;
      return col < F ? Hout + static_cast<int64_t>(row) * F + col : nullptr;
    });
  }
  if constexpr (PHASE == 3 || PHASE == 4) {
    // the gate and up products apart: columns n0.. and F + n0.. of a
    // [rows, 2F] matrix (tile columns 0..127 gate, 128..255 up)
    uint16_t* Gout = static_cast<uint16_t*>(PHASE == 4 ? a.ab : a.H) +
                     static_cast<int64_t>(hrow0) * 2 * a.F;
    __syncthreads();
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * WR + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const int col = (ni / (NB / 2)) * 128 + wn * (128 / WN) + (ni % (NB / 2)) * 32 + (lane & 31);
          stage_put<256, false>(stg, row, col, acc[mi][ni][v]);
        }
    __syncthreads();
    const int F = a.F;
    stage_copy_out<BMT, 256, NTHR>(stg, tid, mrows, [&](int row, int ch) -> uint16_t* {
      const int half = ch >> 4;
      const int col = n0 + (ch & 15) * 8;
      return col < F ? Gout + static_cast<int64_t>(row) * 2 * F + half * F + col : nullptr;
    });
  }
  if constexpr (PHASE == 2 || PHASE == 5) {
    uint16_t* Yout = routed ? static_cast<uint16_t*>(a.y_perm) + static_cast<int64_t>(arow0) * a.d
                            : static_cast<uint16_t*>(a.y_shared) +
                                  static_cast<int64_t>(hrow0 - a.T * a.k) * a.d;
    __syncthreads();
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * WR + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const int col = wn * (kBN2 / WN) + ni * 32 + (lane & 31);
          stage_put<256, PHASE == 2>(stg, row, col, acc[mi][ni][v]);
        }
    __syncthreads();
    const int ld = a.d;
    stage_copy_out<BMT, 256, NTHR>(stg, tid, mrows, [&](int row, int ch) -> uint16_t* {
      const int col = n0 + ch * 8;
      return col < N ? Yout + static_cast<int64_t>(row) * ld + col : nullptr;
    });
  }
}

// The configuration the library launches: K slices of 64, four wavefronts
// of 128 x 128 with the mid-slice barrier for every phase; the K-contiguous
// forms (phases 1-4, and the weight gradients when their offsets fit 32
// bits) on the ring of five operand parts, the MN-contiguous one (phase 5)
// on a ring of two slices (kNSTsel), as is the weight gradients' fallback
// of eight wavefronts of 128 x 64.
constexpr int kBKsel = 64;
constexpr int kNSTsel = 2;
constexpr int kWavesSel = 8;       // wgrad fallback for offsets past 32 bits
constexpr int kBigWaves = 4;

// The dynamic LDS above the default limit is a per-device setting of a
// kernel: set it once for each (kernel, device) the process launches on.
template <auto Kern>
hipError_t allow_dynamic_lds(int bytes) {
  static std::atomic<uint64_t> done{0};        // one bit per device id < 64
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  err = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (err == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
  return err;
}

template <int PHASE>
hipError_t launch_gemm_big(const FfnArgs& a, int nt, int64_t mt, int ncu, hipStream_t s) {
  // whole-tile blocks (at most every tile, in XCD-sized steps) plus one
  // wave of split-K blocks
  const int64_t lmax = mt * nt;
  const unsigned g = static_cast<unsigned>(kXcds * ((lmax + kXcds - 1) / kXcds) + ncu);
  constexpr int kBK = kBKsel, kNST = PHASE == 5 ? kNSTsel : 5;
  constexpr size_t lds = static_cast<size_t>(ring_bytes<kBK, kBM2, kNST>());
  static_assert(lds <= 160 * 1024, "LDS ring exceeds the 160 KB of a CU");
  constexpr int kWaves = kBigWaves;
  constexpr auto kern = &gemm_big_kernel<PHASE, kBK, kNST, kWaves, kBM2, kWM>;
  const hipError_t attr = allow_dynamic_lds<kern>(static_cast<int>(lds));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(g), dim3(kWaves * kWave), lds, s, a, nt, ncu);
  return hipGetLastError();
}

// ------------------------------------------------------------- fp32 VALU --

// Tile: 64 rows x 64 B-rows, K step 16; thread (ty, tx) = (tid / 16,
// tid % 16) owns rows ty*4 .. ty*4+3.  Phase 1: B-rows 0..31 are W1
// columns n0..n0+31 and 32..63 the same W3 columns; the thread owns H
// columns tx*2, tx*2+1 (gate and up).  Phase 2: columns tx*4 .. tx*4+3.
template <int PHASE>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(FfnArgs a) {
  constexpr int BKf = 16;
  __shared__ float As[kBMf][BKf + 1];
  __shared__ float Bs[64][BKf + 1];
  if (static_cast<int>(blockIdx.x) >= *a.ntiles) return;
  const int4 tl = a.tiles[blockIdx.x];
  const int seg = tile_seg(tl.x), arow0 = tl.y, mrows = tl.z, hrow0 = tl.w;
  const bool routed = seg < a.E;
  const int e = routed ? seg : seg - a.E;
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  const int K = PHASE == 1 ? a.d : a.F;
  const int N = PHASE == 1 ? a.F : a.d;
  const int n0 = blockIdx.y * (PHASE == 1 ? 32 : 64);
  const float* A = PHASE == 1
      ? static_cast<const float*>(routed ? a.x_perm : a.x) + static_cast<int64_t>(arow0) * K
      : static_cast<const float*>(a.H) + static_cast<int64_t>(hrow0) * K;
  const int64_t wstride = static_cast<int64_t>(a.F) * a.d;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += BKf) {
    // 64 x 16 of A and of B: 1024 values each, 4 per thread.
    for (int q = tid; q < 64 * BKf; q += kThreads) {
      const int r = q / BKf, c = q % BKf;
      As[r][c] = (r < mrows && k0 + c < K) ? A[static_cast<int64_t>(r) * K + k0 + c] : 0.f;
      float bv = 0.f;
      int col;
      const float* W;
      if (PHASE == 1) {
        col = n0 + (r & 31);
        W = static_cast<const float*>(r < 32 ? (routed ? a.w1 : a.ws1) : (routed ? a.w3 : a.ws3));
      } else {
        col = n0 + r;
        W = static_cast<const float*>(routed ? a.w2 : a.ws2);
      }
      if (col < N && k0 + c < K) bv = W[e * wstride + static_cast<int64_t>(col) * K + k0 + c];
      Bs[r][c] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < BKf; ++c) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[ty * 4 + i][c];
      if (PHASE == 1) {
        bv[0] = Bs[tx * 2][c];      bv[1] = Bs[tx * 2 + 1][c];
        bv[2] = Bs[32 + tx * 2][c]; bv[3] = Bs[32 + tx * 2 + 1][c];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = Bs[tx * 4 + j][c];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  if (PHASE == 1) {
    float* Hout = static_cast<float*>(a.H) + static_cast<int64_t>(hrow0) * a.F;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = ty * 4 + i;
      if (row >= mrows) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + tx * 2 + j;
        if (col < N) {
          const float g = acc[i][j];
          Hout[static_cast<int64_t>(row) * a.F + col] = (g / (1.0f + expf(-g))) * acc[i][2 + j];
        }
      }
    }
  } else {
    float* Yout = routed ? static_cast<float*>(a.y_perm) + static_cast<int64_t>(arow0) * a.d
                         : static_cast<float*>(a.y_shared) +
                               static_cast<int64_t>(hrow0 - a.T * a.k) * a.d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = ty * 4 + i;
      if (row >= mrows) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx * 4 + j;
        if (col < N) Yout[static_cast<int64_t>(row) * a.d + col] = acc[i][j];
      }
    }
  }
}

// ------------------------------------------------- weight gradients --
//
// C_s[M, N] (fp32) = A_s[M, K_s] B_s[N, K_s]^T for every segment s (routed
// experts, then shared), from K-major copies of the backward's activations:
// A and B are [rows][ld] with segment s in columns poff[s] .. poff[s+1]
// (its rows, zero-padded to a multiple of 64).  256 x 256 tiles, the LDS
// ring main loop of the forward; one block per (segment, tile), all of K.
struct WgradArgs {
  const uint16_t* A;
  const uint16_t* B;
  int64_t ld;
  const int* poff;          // [nseg + 1]
  float* C_routed;          // segment s < E: C_routed + s * M * N
  float* C_shared;          // segment s >= E: C_shared + (s - E) * M * N
  int M, N, E, NT;
};

// WAVES = 4 (NST = 5) runs gemm_mainloop_p5 through buffer resources (the
// tile's rows then lie within 2^31 bytes: ld < 2^22); WAVES = 8 (NST = 2)
// the barrier-per-slice loop on 64-bit addresses.
template <int BKT, int NST, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4)))
void gemm_wgrad_kernel(WgradArgs a) {
  constexpr bool kMid = WAVES == 4;
  constexpr int BMT = 256;
  using G = SliceGeom<BKT, BMT>;
  constexpr int WN = WAVES / 2;
  constexpr int WR = BMT / 2;
  constexpr int MI = WR / 32;
  constexpr int NB = kBN2 / WN / 32;
  constexpr int AROWS = BMT / WAVES;
  constexpr int BROWS = kBN2 / WAVES;
  constexpr int NIA = AROWS / G::RPI;
  constexpr int NIB = BROWS / G::RPI;
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];

  const int seg = blockIdx.y;
  const int mt = blockIdx.x / a.NT, nt = blockIdx.x % a.NT;
  const int m0 = mt * BMT, n0 = nt * kBN2;
  const int k0 = a.poff[seg];
  const int nk = (a.poff[seg + 1] - k0) / BKT;
  float* C = seg < a.E ? a.C_routed + static_cast<int64_t>(seg) * a.M * a.N
                       : a.C_shared + static_cast<int64_t>(seg - a.E) * a.M * a.N;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave-uniform by construction; readfirstlane lets the compiler keep it
  // (and the buffer resources chosen by it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / WN, wn = wave % WN;

  const uint16_t* asrc[NIA];
  const uint16_t* bsrc[NIB];
#pragma unroll
  for (int i = 0; i < NIA; ++i) {
    const int r = wave * AROWS + i * G::RPI + lane / G::CH;
    const int lchunk = (lane % G::CH) ^ ((r / G::RPL) % G::CH);
    const int row = min(m0 + r, a.M - 1);
    asrc[i] = a.A + static_cast<int64_t>(row) * a.ld + k0 + lchunk * 8;
  }
#pragma unroll
  for (int i = 0; i < NIB; ++i) {
    const int r = wave * BROWS + i * G::RPI + lane / G::CH;
    const int lchunk = (lane % G::CH) ^ ((r / G::RPL) % G::CH);
    const int row = min(n0 + r, a.N - 1);
    bsrc[i] = a.B + static_cast<int64_t>(row) * a.ld + k0 + lchunk * 8;
  }
  char* lds_bytes = reinterpret_cast<char*>(lds);
  const int a_dst = wave * AROWS * G::ROW;
  const int b_dst = BMT * G::ROW + wave * BROWS * G::ROW;
  f32x16_t acc[MI][NB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int jn = 0; jn < NB; ++jn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jn][v] = 0.f;
  int a_off[MI], b_off[NB];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) a_off[mi] = (wm * WR + mi * 32 + (lane & 31)) * G::ROW;
#pragma unroll
  for (int ni = 0; ni < NB; ++ni)
    b_off[ni] = BMT * G::ROW + (wn * (kBN2 / WN) + ni * 32 + (lane & 31)) * G::ROW;
  if constexpr (kMid) {
    static_assert(BKT == 64 && NST == 5, "the five-part ring");
    BufOperands bo;
    bo.ra = buffer_rsrc(a.A + static_cast<int64_t>(m0) * a.ld + k0);
    bo.rb = buffer_rsrc(a.B + static_cast<int64_t>(n0) * a.ld + k0);
    uint32_t aoff[NIA], boff[NIB];
#pragma unroll
    for (int i = 0; i < NIA; ++i)
      aoff[i] = static_cast<uint32_t>((asrc[i] - (a.A + static_cast<int64_t>(m0) * a.ld + k0)) * 2);
#pragma unroll
    for (int i = 0; i < NIB; ++i)
      boff[i] = static_cast<uint32_t>((bsrc[i] - (a.B + static_cast<int64_t>(n0) * a.ld + k0)) * 2);
    if (nk > 0)
      gemm_mainloop_p5<BKT, BMT, NIA, NIB, MI, NB, MI>(acc, lds_bytes, a_dst, b_dst, a_off, b_off,
                                                         lane, nk, bo, aoff, boff);
  } else {
    if (nk > 0)
      gemm_mainloop<BKT, BMT, NST, NIA, NIB, MI, NB, MI, false>(acc, asrc, bsrc, lds_bytes, a_dst,
                                                                b_dst, a_off, b_off, lane, nk, 1,
                                                                1 << 30, 0);
  }
  // (a segment with no rows stores zeros)
#pragma unroll
  for (int ni = 0; ni < NB; ++ni) {
    const int col = n0 + wn * (kBN2 / WN) + ni * 32 + (lane & 31);
    if (col >= a.N) continue;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * WR + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        // non-temporal: the fp32 gradient is written once and not re-read
        // here (1.5% faster backward on the Mixtral layer)
        if (row < a.M)
          __builtin_nontemporal_store(acc[mi][ni][v], &C[static_cast<int64_t>(row) * a.N + col]);
      }
  }
}

hipError_t launch_wgrad(const WgradArgs& a0, int nseg, hipStream_t s) {
  WgradArgs a = a0;
  a.NT = (a.N + kBN2 - 1) / kBN2;
  const int MT = (a.M + 255) / 256;
  constexpr size_t lds = static_cast<size_t>(kNSTsel) * SliceGeom<kBKsel, 256>::STAGE;
  const dim3 grid(static_cast<unsigned>(MT * a.NT), static_cast<unsigned>(nseg));
  if (a.ld < (int64_t(1) << 22)) {
    // a tile's 256 rows of ld bf16 fit the 32-bit offsets of a buffer load
    constexpr auto kern = &gemm_wgrad_kernel<kBKsel, 5, kBigWaves>;
    constexpr size_t lds5 = ring_bytes<kBKsel, 256, 5>();
    const hipError_t attr = allow_dynamic_lds<kern>(static_cast<int>(lds5));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, grid, dim3(kBigWaves * kWave), lds5, s, a);
  } else {
    constexpr auto kern = &gemm_wgrad_kernel<kBKsel, kNSTsel, kWavesSel>;
    const hipError_t attr = allow_dynamic_lds<kern>(static_cast<int>(lds));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, grid, dim3(kWavesSel * kWave), lds, s, a);
  }
  return hipGetLastError();
}

int64_t max_tiles(int64_t T, int E, int Es, int k, int BM) {
  return (T * k + BM - 1) / BM + E + static_cast<int64_t>(Es) * ((T + BM - 1) / BM);
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

// Workspace: tile count and table, the bf16 split-K partial tiles and
// arrival counters, then the intermediate H.
size_t ffn_sk_bytes(int elem_bytes) {
  return elem_bytes == 2 ? static_cast<size_t>(kMaxCUs) * kBM2 * kBN2 * sizeof(float) +
                               align256(2 * kMaxCUs * sizeof(unsigned))
                         : 0;
}

size_t ffn_workspace_bytes(int64_t T, int E, int E_shared, int k, int64_t d_ff,
                           int elem_bytes) {
  const int64_t tiles = max_tiles(T, E, E_shared, k, kBMf);   // the smaller BM bounds both
  const int64_t hrows = T * k + static_cast<int64_t>(E_shared) * T;
  return 256 + align256(static_cast<size_t>(tiles) * sizeof(int4)) + ffn_sk_bytes(elem_bytes) +
         static_cast<size_t>(hrows) * d_ff * elem_bytes;
}

namespace {

// Rows per tile of the path launch_expert_ffn takes for this shape: the
// fp32 tiles, the large bf16 tiles (prefill-sized segments) or the 128-row
// bf16 tiles beside the weight-streaming kernels (decode-sized calls).
int ffn_tile_rows(int64_t T, int E, int k, bool bf16) {
  return !bf16 ? kBMf : (T * k >= 64LL * E ? kBM2 : kBM);
}

}  // namespace

// The part of the workspace launch_expert_ffn touches: the tile count and
// table, the split-K partials and arrival counters (large-tile path only),
// then H.  At most ffn_workspace_bytes.
size_t ffn_workspace_used_bytes(int64_t T, int E, int E_shared, int k, int64_t d_ff,
                                int elem_bytes) {
  const bool bf16 = elem_bytes == 2;
  const int64_t tiles = max_tiles(T, E, E_shared, k, kBMf);
  const int64_t hrows = T * k + static_cast<int64_t>(E_shared) * T;
  const bool big = bf16 && ffn_tile_rows(T, E, k, bf16) == kBM2;
  return 256 + align256(static_cast<size_t>(tiles) * sizeof(int4)) +
         (big ? ffn_sk_bytes(2) : 0) + static_cast<size_t>(hrows) * d_ff * elem_bytes;
}

namespace {

// Compute units of the current device (one large-tile block fits a CU).
hipError_t device_cus(int* ncu) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess)
    err = hipDeviceGetAttribute(ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (err == hipSuccess) *ncu = max(kXcds, min(*ncu, kMaxCUs));
  return err;
}

// Both phases on the large tiles (the tile table has been built with
// BM = kBM2); P1 = 1 (H only) or 4 (H and the pre-activations).
template <int P1>
hipError_t run_big_ffn(const FfnArgs& a, hipStream_t s) {
  const int nt1 = (a.F + kBN2 / 2 - 1) / (kBN2 / 2);
  const int nt2 = (a.d + kBN2 - 1) / kBN2;
  const int64_t mt = max_tiles(a.T, a.E, a.Es, a.k, kBM2);
  int ncu = 0;
  hipError_t err = device_cus(&ncu);
  if (err != hipSuccess) return err;
  err = launch_gemm_big<P1>(a, nt1, mt, ncu, s);
  if (err != hipSuccess) return err;
  return launch_gemm_big<2>(a, nt2, mt, ncu, s);
}

}  // namespace

hipError_t launch_expert_ffn_train(int64_t T, int64_t d, int E, int E_shared, int k, int64_t F,
                                   const void* x_perm, const int32_t* offsets, const void* x,
                                   const void* w1, const void* w3, const void* w2,
                                   const void* ws1, const void* ws3, const void* ws2,
                                   void* y_perm, void* y_shared, void* ab, void* ws,
                                   hipStream_t s) {
  char* base = static_cast<char*>(ws);
  int* ntiles = reinterpret_cast<int*>(base);
  int4* tiles = reinterpret_cast<int4*>(base + 256);
  const int64_t tiles_cap = max_tiles(T, E, E_shared, k, kBMf);
  char* sk = base + 256 + align256(static_cast<size_t>(tiles_cap) * sizeof(int4));
  float* sk_partial = reinterpret_cast<float*>(sk);
  unsigned* sk_count =
      reinterpret_cast<unsigned*>(sk + static_cast<size_t>(kMaxCUs) * kBM2 * kBN2 * 4);
  void* H = sk + ffn_sk_bytes(2);
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(kTableThreads), 0, s, offsets, tiles, ntiles, E,
                     E_shared, static_cast<int>(T), k, kBM2, sk_count);
  FfnArgs a{x_perm, x, offsets, w1, w3, w2, ws1, ws3, ws2, H, y_perm, y_shared, tiles, ntiles,
            sk_partial, sk_count,
            static_cast<int>(T), static_cast<int>(d), E, E_shared, k, static_cast<int>(F), ab};
  hipError_t err = run_big_ffn<4>(a, s);
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

hipError_t launch_expert_ffn(int64_t T, int64_t d, int E, int E_shared, int k, int64_t F,
                             bool bf16, const void* x_perm, const int32_t* offsets,
                             const void* x, const void* w1, const void* w3, const void* w2,
                             const void* ws1, const void* ws3, const void* ws2, void* y_perm,
                             void* y_shared, void* ws, hipStream_t s) {
  // Large segments take the large tiles; decode-sized ones (few rows
  // per expert) the 128-row tiles.  Only the large-tile path has split-K
  // partials; H follows the tile table directly on the others
  // (ffn_workspace_used_bytes).
  const int BM = ffn_tile_rows(T, E, k, bf16);
  const bool big = bf16 && BM == kBM2;
  char* base = static_cast<char*>(ws);
  int* ntiles = reinterpret_cast<int*>(base);
  int4* tiles = reinterpret_cast<int4*>(base + 256);
  const int64_t tiles_cap = max_tiles(T, E, E_shared, k, kBMf);
  char* sk = base + 256 + align256(static_cast<size_t>(tiles_cap) * sizeof(int4));
  float* sk_partial = big ? reinterpret_cast<float*>(sk) : nullptr;
  unsigned* sk_count =
      big ? reinterpret_cast<unsigned*>(sk + static_cast<size_t>(kMaxCUs) * kBM2 * kBN2 * 4)
          : nullptr;
  void* H = sk + (big ? ffn_sk_bytes(2) : 0);
  // decode-sized calls with T <= kStreamMaxRows only stream (no tiles)
  const bool stream_only = bf16 && BM == kBM && T <= kStreamMaxRows;
  if (!stream_only)
    hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(kTableThreads), 0, s, offsets, tiles, ntiles, E,
                       E_shared, static_cast<int>(T), k, BM, sk_count);
  FfnArgs a{x_perm, x, offsets, w1, w3, w2, ws1, ws3, ws2, H, y_perm, y_shared, tiles, ntiles,
            sk_partial, sk_count,
            static_cast<int>(T), static_cast<int>(d), E, E_shared, k, static_cast<int>(F)};
  const unsigned gx = static_cast<unsigned>(max_tiles(T, E, E_shared, k, BM));
  if (big) {
    hipError_t err = run_big_ffn<1>(a, s);
    if (err != hipSuccess) return err;
  } else if (bf16) {
    // Decode-sized: segments of at most kStreamMaxRows rows stream their
    // weights; larger ones (possible only when T exceeds that) take the
    // 128-row tiles.
    const bool tiled = !stream_only;
    hipError_t err = launch_ffn_stream(1, T, d, E, E_shared, k, F, x_perm, offsets, x, w1, w3, w2,
                                       ws1, ws3, ws2, H, y_perm, y_shared, s);
    if (err != hipSuccess) return err;
    if (tiled)
      hipLaunchKernelGGL(gemm_bf16_kernel<1>, dim3(gx, static_cast<unsigned>((F + 63) / 64)),
                         dim3(kThreads), 0, s, a);
    err = launch_ffn_stream(2, T, d, E, E_shared, k, F, x_perm, offsets, x, w1, w3, w2, ws1, ws3,
                            ws2, H, y_perm, y_shared, s);
    if (err != hipSuccess) return err;
    if (tiled)
      hipLaunchKernelGGL(gemm_bf16_kernel<2>, dim3(gx, static_cast<unsigned>((d + 127) / 128)),
                         dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(gemm_f32_kernel<1>, dim3(gx, static_cast<unsigned>((F + 31) / 32)),
                       dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(gemm_f32_kernel<2>, dim3(gx, static_cast<unsigned>((d + 63) / 64)),
                       dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- backward --

namespace {

// Workspace of the backward, after the forward's tile table and split-K
// region: segment info, the (A, B) -> (dA, dB) buffer, dH -> H, and the
// K-major copies of X, dO, H and (dA, dB) for the weight gradients.
struct BwdLayout {
  size_t seg, g13, dh, xt, dot, ht, dabt, total;
  int64_t rows, ld;       // H-indexed rows; K-major row length (padded)
};

BwdLayout bwd_layout(int64_t T, int64_t d, int E, int Es, int k, int64_t F) {
  BwdLayout L;
  const int64_t tiles_cap = max_tiles(T, E, Es, k, kBMf);
  size_t at = 256 + align256(static_cast<size_t>(tiles_cap) * sizeof(int4)) + ffn_sk_bytes(2);
  L.rows = T * k + static_cast<int64_t>(Es) * T;
  L.ld = (L.rows + 64LL * (E + Es) + 63) / 64 * 64;
  const int G = E + Es;
  auto take = [&](size_t bytes) { const size_t p = at; at += align256(bytes); return p; };
  L.seg = take(3 * sizeof(int) * (G + 1));
  L.g13 = take(static_cast<size_t>(L.rows) * 2 * F * 2);
  L.dh = take(static_cast<size_t>(L.rows) * F * 2);
  L.xt = take(static_cast<size_t>(d) * L.ld * 2);
  L.dot = take(static_cast<size_t>(d) * L.ld * 2);
  L.ht = take(static_cast<size_t>(F) * L.ld * 2);
  L.dabt = take(static_cast<size_t>(2 * F) * L.ld * 2);
  L.total = at;
  return L;
}

}  // namespace

size_t ffn_backward_workspace_bytes(int64_t T, int64_t d, int E, int E_shared, int k,
                                    int64_t d_ff) {
  return bwd_layout(T, d, E, E_shared, k, d_ff).total;
}

hipError_t launch_expert_ffn_backward(int64_t T, int64_t d, int E, int E_shared, int k,
                                      int64_t F, const void* x_perm, const int32_t* offsets,
                                      const void* x, const void* w1, const void* w3,
                                      const void* w2, const void* ws1, const void* ws3,
                                      const void* ws2, const void* dy_perm, void* dx_perm,
                                      void* dx_shared, float* dw1, float* dw3, float* dw2,
                                      float* dws1, float* dws3, float* dws2, const void* ab,
                                      void* ws, hipStream_t s) {
  const BwdLayout L = bwd_layout(T, d, E, E_shared, k, F);
  char* base = static_cast<char*>(ws);
  int* ntiles = reinterpret_cast<int*>(base);
  int4* tiles = reinterpret_cast<int4*>(base + 256);
  const int64_t tiles_cap = max_tiles(T, E, E_shared, k, kBMf);
  char* sk = base + 256 + align256(static_cast<size_t>(tiles_cap) * sizeof(int4));
  float* sk_partial = reinterpret_cast<float*>(sk);
  unsigned* sk_count =
      reinterpret_cast<unsigned*>(sk + static_cast<size_t>(kMaxCUs) * kBM2 * kBN2 * 4);
  const int G = E + E_shared;
  int* poff = reinterpret_cast<int*>(base + L.seg);
  int* hstart = poff + (G + 1);
  int* nrows = hstart + (G + 1);
  void* g13 = base + L.g13;
  void* dh = base + L.dh;
  const int Fi = static_cast<int>(F), di = static_cast<int>(d);

  hipError_t err = hipSuccess;
  auto ok = [&](hipError_t e) { if (err == hipSuccess) err = e; return err == hipSuccess; };
  // tiles of the large-tile kernel (and zeroed split-K counters), segment info
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(kTableThreads), 0, s, offsets, tiles, ntiles, E,
                     E_shared, static_cast<int>(T), k, kBM2, sk_count);
  ok(launch_seg_info(offsets, poff, hstart, nrows, E, E_shared, T, k, s));
  int ncu = 0;
  if (!ok(device_cus(&ncu))) return err;
  const int64_t mt = max_tiles(T, E, E_shared, k, kBM2);
  auto nt_of = [](int64_t n, int cols) { return static_cast<int>((n + cols - 1) / cols); };
  // 1. A = X W1^T and B = X W3^T: kept by the forward (ab), else recomputed
  //    into the (A, B) rows of g13
  if (ab == nullptr) {
    FfnArgs a3{x_perm, x, offsets, w1, w3, w2, ws1, ws3, ws2, g13, nullptr, nullptr, tiles,
               ntiles, sk_partial, sk_count, static_cast<int>(T), di, E, E_shared, k, Fi};
    ok(launch_gemm_big<3>(a3, nt_of(F, kBN2 / 2), mt, ncu, s));
  }
  // 2. dH = dO W2: the phase-2 form with K = d and N = F, reading the
  //    rows of W2 [d, F] as stored (PHASE 5)
  FfnArgs ah{nullptr, nullptr, offsets, nullptr, w2, w2, nullptr, ws2, ws2,
             const_cast<void*>(dy_perm), dh, static_cast<uint16_t*>(dh) + T * k * F, tiles,
             ntiles, sk_partial, sk_count, static_cast<int>(T), Fi, E, E_shared, k, di,
             nullptr, di};
  ok(launch_gemm_big<5>(ah, nt_of(F, kBN2), mt, ncu, s));
  // 3. (A, B), dH -> (dA, dB) row-major in g13, and the K-major copies
  //    dA^T, dB^T, H^T the weight gradients read
  uint16_t* xt = reinterpret_cast<uint16_t*>(base + L.xt);
  uint16_t* dot = reinterpret_cast<uint16_t*>(base + L.dot);
  uint16_t* ht = reinterpret_cast<uint16_t*>(base + L.ht);
  uint16_t* dabt = reinterpret_cast<uint16_t*>(base + L.dabt);
  ok(launch_swiglu_bwd_t(ab != nullptr ? ab : g13, g13, dh, dabt, ht, poff, hstart, nrows, E,
                         E_shared, T, F, L.ld, s));
  // 4. dX = [dA dB] [W1; W3]: the phase-2 form with K = 2F and N = d, B
  //    rows from W1 [F, d] then W3 [F, d] as stored (PHASE 5)
  FfnArgs ax{nullptr, nullptr, offsets, nullptr, w3, w1, nullptr, ws3, ws1, g13, dx_perm,
             dx_shared, tiles, ntiles, sk_partial, sk_count, static_cast<int>(T), di, E,
             E_shared, k, 2 * Fi, nullptr, Fi};
  ok(launch_gemm_big<5>(ax, nt_of(d, kBN2), mt, ncu, s));
  // 5. K-major copies of X and dO for the weight gradients
  ok(launch_transpose_seg(x_perm, x, xt, poff, hstart, nrows, di, L.ld, E, E_shared, T, k, s));
  ok(launch_transpose_seg(dy_perm, nullptr, dot, poff, hstart, nrows, di, L.ld, E, E_shared, T,
                          k, s));
  // 6. dW1 = dA^T X, dW3 = dB^T X  ([F, d]),  dW2 = dO^T H  ([d, F])
  WgradArgs g1{dabt, xt, L.ld, poff, dw1, dws1, Fi, di, E, 0};
  ok(launch_wgrad(g1, G, s));
  WgradArgs g3{dabt + F * L.ld, xt, L.ld, poff, dw3, dws3, Fi, di, E, 0};
  ok(launch_wgrad(g3, G, s));
  WgradArgs g2{dot, ht, L.ld, poff, dw2, dws2, di, Fi, E, 0};
  ok(launch_wgrad(g2, G, s));
  return err;
}

}  // namespace moe
