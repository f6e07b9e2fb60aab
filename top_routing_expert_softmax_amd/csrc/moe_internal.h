// Host-side launchers behind the C ABI.  Arguments are validated by the
// caller (moe_api.hip); these only size grids and enqueue kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Token chunking shared by the dispatch kernels: blocks of kDispatchThreads
// threads, at most kMaxDispatchBlocks blocks (so the per-expert scan over
// blocks fits one wavefront).
constexpr int kDispatchThreads = 256;
constexpr int kMaxDispatchBlocks = 64;

// Statistics: at most this many partial blocks.
constexpr int kStatsBlocks = 256;

// Expert choice: at most this many tokens per expert (the picks of one
// expert are sorted in LDS).
constexpr int kEcMaxCap = 4096;

// Decode-sized expert segments (at most this many rows) take the
// weight-streaming FFN kernels.
constexpr int kStreamMaxRows = 64;

size_t route_workspace_bytes(int64_t T, int64_t d, int E);
size_t permute_workspace_bytes(int64_t T, int E);
size_t stats_workspace_bytes(int64_t T, int E);
size_t ffn_workspace_bytes(int64_t T, int E, int E_shared, int k, int64_t d_ff,
                           int elem_bytes);
size_t ffn_workspace_used_bytes(int64_t T, int E, int E_shared, int k, int64_t d_ff,
                                int elem_bytes);

struct GateParams;   // router.hip: which top-k follows the logits

hipError_t launch_route(int64_t T, int64_t d, int E, int k, bool bf16,
                        const void* x, const void* w_gate, float* logits,
                        int32_t* topk_idx, float* topk_w, void* ws,
                        const GateParams& gp, hipStream_t s);

// The softmax top-k router and the DeepSeek-V3 gate.
hipError_t launch_route_softmax(int64_t T, int64_t d, int E, int k, bool bf16,
                                const void* x, const void* w_gate, float* logits,
                                int32_t* topk_idx, float* topk_w, void* ws,
                                hipStream_t s);
hipError_t launch_route_v3(int64_t T, int64_t d, int E, int k, int n_groups,
                           int topk_groups, float route_scale, bool bf16,
                           const void* x, const void* w_gate, const float* bias,
                           float* logits, int32_t* topk_idx, float* topk_w,
                           void* ws, hipStream_t s);
hipError_t launch_update_bias(int64_t T, int E, int k, float gamma,
                              const int32_t* counts, float* bias, hipStream_t s);
// Logits only (no top-k).
hipError_t launch_logits(int64_t T, int64_t d, int E, bool bf16, const void* x,
                         const void* w_gate, float* logits, void* ws, hipStream_t s);

// Expert choice (ec.hip).
size_t ec_workspace_bytes(int64_t T, int64_t d, int E);
hipError_t launch_route_ec(int64_t T, int64_t d, int E, int64_t cap, bool bf16,
                           const void* x, const void* w_gate, float* logits,
                           int32_t* ec_token, float* ec_w, void* ws, hipStream_t s);
hipError_t launch_permute_ec(int64_t T, int64_t d, int E, int64_t cap, bool bf16,
                             const int32_t* ec_token, const float* ec_w,
                             const void* x, int32_t* offsets, int32_t* row_of_te,
                             float* w_te, void* x_perm, hipStream_t s);

hipError_t launch_permute(int64_t T, int64_t d, int E, int k, int64_t cap,
                          bool bf16, const int32_t* topk_idx, const void* x,
                          int32_t* counts, int32_t* offsets,
                          int32_t* token_of_row, int32_t* row_of_pair,
                          uint8_t* drop_mask, void* x_perm, void* ws,
                          hipStream_t s);

hipError_t launch_expert_ffn(int64_t T, int64_t d, int E, int E_shared, int k,
                             int64_t F, bool bf16, const void* x_perm,
                             const int32_t* offsets, const void* x,
                             const void* w1, const void* w3, const void* w2,
                             const void* ws1, const void* ws3, const void* ws2,
                             void* y_perm, void* y_shared, void* ws,
                             hipStream_t s);
// The bf16 forward on the large tiles that also stores the pre-activations
// A = X W1^T and B = X W3^T of every H row to ab [rows, 2F].
hipError_t launch_expert_ffn_train(int64_t T, int64_t d, int E, int E_shared, int k, int64_t F,
                                   const void* x_perm, const int32_t* offsets, const void* x,
                                   const void* w1, const void* w3, const void* w2,
                                   const void* ws1, const void* ws3, const void* ws2,
                                   void* y_perm, void* y_shared, void* ab, void* ws,
                                   hipStream_t s);

// One phase (1: H = SiLU(X W1^T) * (X W3^T), 2: Y = H W2^T) of the
// weight-streaming FFN over the segments with 1 .. kStreamMaxRows rows.
// With row scales (sc1 non-null) the weights are FP8 E4M3 codes.
hipError_t launch_ffn_stream(int phase, int64_t T, int64_t d, int E, int E_shared, int k,
                             int64_t F, const void* x_perm, const int32_t* offsets,
                             const void* x, const void* w1, const void* w3, const void* w2,
                             const void* ws1, const void* ws3, const void* ws2, void* H,
                             void* y_perm, void* y_shared, hipStream_t s,
                             const float* sc1 = nullptr, const float* sc3 = nullptr,
                             const float* sc2 = nullptr, const float* ssc1 = nullptr,
                             const float* ssc3 = nullptr, const float* ssc2 = nullptr);

// Expert-FFN backward (ffn.hip orchestrates; helpers in ffn_bwd.hip).
size_t ffn_backward_workspace_bytes(int64_t T, int64_t d, int E, int E_shared, int k,
                                    int64_t d_ff);
hipError_t launch_expert_ffn_backward(int64_t T, int64_t d, int E, int E_shared, int k,
                                      int64_t F, const void* x_perm, const int32_t* offsets,
                                      const void* x, const void* w1, const void* w3,
                                      const void* w2, const void* ws1, const void* ws3,
                                      const void* ws2, const void* dy_perm, void* dx_perm,
                                      void* dx_shared, float* dw1, float* dw3, float* dw2,
                                      float* dws1, float* dws3, float* dws2, const void* ab,
                                      void* ws, hipStream_t s);
hipError_t launch_seg_info(const int32_t* offsets, int* poff, int* hstart, int* nrows, int E,
                           int Es, int64_t T, int k, hipStream_t s);
hipError_t launch_transpose_seg(const void* src, const void* src_shared, void* dst,
                                const int* poff, const int* hstart, const int* nrows, int C,
                                int64_t ld, int E, int Es, int64_t T, int k, hipStream_t s);
hipError_t launch_swiglu_bwd_t(const void* ab, void* g13, const void* dh, void* dabt, void* ht,
                               const int* poff, const int* hstart, const int* nrows, int E,
                               int Es, int64_t T, int64_t F, int64_t ld, hipStream_t s);

// Combine and router backward (bwd.hip).
hipError_t launch_combine_backward(int64_t T, int64_t d, int E_shared, int k, const void* dy,
                                   const void* y_perm, const int32_t* row_of_pair,
                                   const float* topk_w, void* dy_perm, float* dtopk_w,
                                   hipStream_t s);
size_t route_backward_workspace_bytes(int64_t T, int64_t d, int E);
hipError_t launch_route_backward(int64_t T, int64_t d, int E, int E_shared, int k, const void* x,
                                 const void* w_gate, const float* logits,
                                 const int32_t* topk_idx, const float* topk_w,
                                 const float* dtopk_w, const int32_t* counts,
                                 const int32_t* row_of_pair, const void* dx_perm,
                                 const void* dx_shared, float alpha, float beta, void* dx,
                                 float* dw_gate, void* ws, hipStream_t s);

// Per-row FP8 E4M3 quantisation (quant.hip).
hipError_t launch_quantize_fp8(int64_t rows, int64_t cols, bool bf16, const void* w,
                               uint8_t* codes, float* scales, hipStream_t s);

hipError_t launch_combine(int64_t T, int64_t d, int E_shared, int k, bool bf16,
                          const void* y_perm, const void* y_shared,
                          const int32_t* row_of_pair, const float* topk_w,
                          void* y, hipStream_t s);

hipError_t launch_aux_stats(int64_t T, int E, int k, int64_t cap,
                            const float* logits, const int32_t* counts,
                            float* f, float* P, double* scalars, void* ws,
                            hipStream_t s);

}  // namespace moe
