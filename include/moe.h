/*
 * moe.h - C ABI of the MI355X (gfx950) forward pass of one Mixture-of-Experts
 * layer with softmax top-k routing.
 *
 * The layer, in the notation of the pages it follows:
 *   g = x W_gate                                  ("MoE routing math", sec. 2.1)
 *   p = softmax(g);  S = TopK(p, k);  p~_i = p_i / sum_{j in S} p_j   (sec. 2.1)
 *   capacity = ceil(CF * k * T / E), overflow dropped
 *                         ("CMU 11-868 Lecture 17: Systems for MoE Models", 2.4)
 *   group (token, choice) pairs by expert, one product per expert     (L17, 2.2)
 *   Expert(x) = (SiLU(x W1) (*) x W3) W2                              (L17, 5.2)
 *   y = sum_s Shared_s(x) + sum_{i in S, kept} p~_i Expert_i(x)
 *                                            ("MoE routing math", sec. 2.2)
 *   f_i, P_i, L_balance = E sum_i f_i P_i    ("MoE routing math", sec. 3.2)
 *   z = mean_t (logsumexp_i g_ti)^2          ("MoE deep dive: routing and
 *                                              load balancing", sec. 3.2)
 *
 * Notation: T tokens, d = d_model, E routed experts, E_shared always-on
 * shared experts, k experts per token, F = d_ff, CF capacity factor.
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers, row-major and contiguous,
 *     16-byte aligned.  The caller owns every buffer; the library never
 *     allocates, frees or keeps a pointer after the call returns.
 *   - State the library keeps: the last error message, per calling thread
 *     (thread-local); a per-device record of the large-LDS launch attribute
 *     it has set on its GEMM and weight-streaming kernels (set once, under
 *     an atomic); and the
 *     per-device address of the scratch array of moe_expert_ffn_noalloc.
 *     Device state lives only in the caller's workspace (and in that
 *     scratch array): moe_expert_ffn keeps split-K arrival counters and
 *     partial tiles there, so two calls that run at the same time (two
 *     streams, or two threads) need a workspace each.  Calls made one after
 *     another on one stream may share a workspace.
 *   - dtype selects activations AND weights: MOE_F32 (fp32) or MOE_BF16
 *     (bf16 storage).  Accumulation is always fp32.  Router logits,
 *     weights and statistics are fp32 (scalars fp64) for both dtypes.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  All
 *     device work is enqueued on it; outputs are valid once the caller has
 *     synchronised the stream.  No call waits on the device.
 *   - Arguments are checked on the host before anything is launched.  On
 *     error nothing is launched and a negative MOE_E* code is returned;
 *     moe_last_error() then describes it (per calling thread).  A device
 *     fault surfaces at the caller's next synchronisation as a HIP error.
 *   - Limits: 1 <= k <= min(E, 64); E <= 256; 0 <= E_shared <= 16; 1 <= T;
 *     T*k + E_shared*T < 2^31; d_model and d_ff positive multiples of 64
 *     below 2^22 (a 256-row operand tile then spans less than 2^31 bytes,
 *     the reach of the GEMM's 32-bit buffer offsets).
 *   - topk_idx rows must name distinct experts (moe_route writes them so);
 *     ids outside [0, E) are treated as dropped pairs.
 *
 * Weight layouts (each stored row is one output feature's weights along
 * the contracted dimension, the [out, in] layout of a linear layer):
 *   w_gate [d, E]          the pages' W_gate in R^{d x E}
 *   w1, w3 [E, F, d]       w1[e][f][i] = W1_e[i][f]  (W1_e in R^{d x F})
 *   w2     [E, d, F]       w2[e][i][f] = W2_e[f][i]  (W2_e in R^{F x d})
 *   ws1, ws3 [E_shared, F, d];  ws2 [E_shared, d, F]   same, shared experts
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* bad argument: null, misaligned, out of range */
  MOE_EUNSUPPORTED = -2, /* a dtype or shape with no kernel */
  MOE_EHIP = -3,         /* a HIP launch or query failed (message kept) */
  MOE_EWORKSPACE = -4    /* workspace smaller than moe_workspace_size() */
};

enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* Static description of a status code. */
const char* moe_strerror(int status);

/* Message of the last failing call made by this thread ("" if none). */
const char* moe_last_error(void);

/*
 * Expert capacity, "CMU 11-868 Lecture 17", section 2.4:
 *   cap = min(T, ceil(CF * k * T / E)),
 * evaluated exactly on the double value CF (no rounding of the product).
 * A token picks an expert at most once, hence the clamp to T.  CF <= 0
 * means no capacity limit (cap = T).  Host only.  Returns MOE_OK and
 * writes *cap, or MOE_EINVAL.
 */
int moe_capacity(int64_t T, int32_t E, int32_t k, double CF, int64_t* cap);

/*
 * Bytes of device workspace that moe_route, moe_permute, moe_expert_ffn
 * and moe_aux_stats need for this shape (one buffer serves all four; calls
 * that run one after another on one stream may share it, calls that run
 * concurrently need one each).  Host only.
 */
int moe_workspace_size(int64_t T, int64_t d_model, int32_t E, int32_t E_shared,
                       int32_t k, int64_t d_ff, int32_t dtype, size_t* bytes);

/*
 * Router, "MoE routing math" section 2.1: logits g = x W_gate, softmax,
 * top-k and renormalisation.  (The pages also write the weights as a
 * softmax over only the k largest logits; the two are equal.)
 *   x       [T, d]  dtype            in
 *   w_gate  [d, E]  dtype            in
 *   logits  [T, E]  fp32             out  exact when x and W_gate lie on a
 *                                         common dyadic grid whose integer
 *                                         partial sums stay below 2^24
 *   topk_idx[T, k]  int32            out  expert ids, larger logit first,
 *                                         ties to the lower expert id
 *   topk_w  [T, k]  fp32             out  renormalised weights p~ (sum 1)
 *   ws      workspace of moe_workspace_size() bytes (used when T is small
 *           and d is split across blocks; may be NULL otherwise)
 */
int moe_route(int64_t T, int64_t d_model, int32_t E, int32_t k, int32_t dtype,
              const void* x, const void* w_gate, float* logits,
              int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
              void* stream);

/*
 * DeepSeek-V3 gate ("CMU 11-868 Lecture 17" section 5.3, the sigmoid
 * branch of the V3 inference gate; the bias of section 3.4), on the same
 * logits g = x W_gate as moe_route:
 *   s = sigmoid(g)                 per expert (fp64, rounded once to fp32)
 *   biased = s + bias              fp32; the bias only steers the choice
 *   group score = sum of the two largest biased scores of each of n_groups
 *                 contiguous groups of E / n_groups experts (fp32)
 *   keep the topk_groups best groups, then choose the k largest biased
 *   scores among their experts (ties to the lower group / expert index)
 *   topk_w = route_scale * s_j / sum of s over the chosen j
 * (V3: E = 256, n_groups = 8, topk_groups = 4, k = 8, route_scale = 2.5.)
 *   x, w_gate, logits, topk_idx, topk_w, ws: as for moe_route; topk_idx is
 *                 ordered by biased score, larger first
 *   bias   [E]  fp32  in
 * Requires E % n_groups == 0, E / n_groups >= 2, n_groups <= 64,
 * 1 <= topk_groups <= n_groups and k <= topk_groups * E / n_groups.
 * The outputs feed moe_permute and moe_combine unchanged (the weights of a
 * token sum to route_scale).
 */
int moe_route_v3(int64_t T, int64_t d_model, int32_t E, int32_t k,
                 int32_t n_groups, int32_t topk_groups, float route_scale,
                 int32_t dtype, const void* x, const void* w_gate,
                 const float* bias, float* logits, int32_t* topk_idx,
                 float* topk_w, void* ws, size_t ws_bytes, void* stream);

/*
 * Balance-bias step of DeepSeek-V3 ("CMU 11-868 Lecture 17" section 3.4):
 * for each expert e, with the mean load T k / E compared exactly,
 *   counts[e] > mean:  bias[e] -= gamma
 *   counts[e] < mean:  bias[e] += gamma
 *   counts[e] = mean:  unchanged
 *   counts [E] int32 in (pre-drop, from moe_permute); bias [E] fp32 in/out.
 */
int moe_update_bias(int64_t T, int32_t E, int32_t k, float gamma,
                    const int32_t* counts, float* bias, void* stream);

/*
 * Expert choice ("MoE deep dive: routing mechanisms and load balancing",
 * section 2.2): experts pick tokens.  Tokens per expert
 *   cap = min(T, floor((T // E) * CF))       (exact on the double CF)
 * Host only; CF >= 0.
 */
int moe_ec_capacity(int64_t T, int32_t E, double CF, int64_t* cap);

/*
 * Expert-choice router: logits g = x W_gate as in moe_route, then each
 * expert e takes the cap tokens with the largest g[t][e] (larger first, ties
 * to the lower token index).  The weight of a chosen pair is the router
 * probability softmax(g[t])[e] (fp32); it is not renormalised.
 *   x [T, d], w_gate [d, E]  dtype in;  logits [T, E] fp32 out
 *   ec_token [E, cap] int32 out;  ec_w [E, cap] fp32 out
 *   ws: moe_workspace_size() bytes
 * Limits: 0 <= cap <= min(T, 4096); T * E < 2^31.
 */
int moe_route_ec(int64_t T, int64_t d_model, int32_t E, int64_t cap,
                 int32_t dtype, const void* x, const void* w_gate,
                 float* logits, int32_t* ec_token, float* ec_w, void* ws,
                 size_t ws_bytes, void* stream);

/*
 * Grouped layout of the expert-choice picks ("CMU 11-868 Lecture 17" section
 * 2.2, one segment per expert): expert e owns rows e*cap .. e*cap+cap-1.
 *   ec_token, ec_w [E, cap]   in (from moe_route_ec)
 *   x [T, d] dtype            in
 *   offsets [E + 1] int32     out  e * cap
 *   row_of_te [T, E] int32    out  row of (t, e), -1 if e did not pick t
 *   w_te [T, E] fp32          out  weight of (t, e), 0 if e did not pick t
 *   x_perm [E * cap, d] dtype out  row r = x[ec_token[r]]
 * Then moe_expert_ffn runs unchanged with k = ceil(E * cap / T) (its row
 * bound T * k covers the E * cap rows), and moe_combine with k = E,
 * row_of_pair = row_of_te and topk_w = w_te.
 */
int moe_permute_ec(int64_t T, int64_t d_model, int32_t E, int64_t cap,
                   int32_t dtype, const int32_t* ec_token, const float* ec_w,
                   const void* x, int32_t* offsets, int32_t* row_of_te,
                   float* w_te, void* x_perm, void* stream);

/*
 * Counting, capacity, drop and permutation, "CMU 11-868 Lecture 17"
 * sections 2.2 (group by expert) and 2.4 (capacity, overflow dropped).
 * Pairs (t, j) are ranked inside their expert in token order; a pair is
 * kept iff its rank < cap = moe_capacity(T, E, k, CF).
 *   topk_idx     [T, k]     int32   in
 *   x            [T, d]     dtype   in
 *   counts       [E]        int32   out  pairs per expert before the drop
 *   offsets      [E + 1]    int32   out  exclusive scan of min(counts, cap);
 *                                        offsets[E] = R, the kept rows
 *   token_of_row [T * k]    int32   out  token of each kept row, -1 past R
 *   row_of_pair  [T, k]     int32   out  row of pair (t, j), -1 if dropped
 *   drop_mask    [T, k]     uint8   out  1 if pair (t, j) was dropped
 *   x_perm       [T * k, d] dtype   out  rows 0..R-1 = x[token_of_row[r]];
 *                                        rows >= R are not written
 * Rows are sorted by (expert, token).  Needs ws of moe_workspace_size().
 */
int moe_permute(int64_t T, int64_t d_model, int32_t E, int32_t k, double CF,
                int32_t dtype, const int32_t* topk_idx, const void* x,
                int32_t* counts, int32_t* offsets, int32_t* token_of_row,
                int32_t* row_of_pair, uint8_t* drop_mask, void* x_perm,
                void* ws, size_t ws_bytes, void* stream);

/*
 * Grouped expert FFN, "CMU 11-868 Lecture 17" sections 2.2 and 5.2: for
 * each routed expert e, its kept rows x_perm[offsets[e] .. offsets[e+1])
 * go through (SiLU(X W1_e) (*) X W3_e) W2_e; each shared expert s
 * ("MoE routing math" section 2.2) takes all T rows of x.
 *   x_perm   [T * k, d]        dtype  in   (rows past offsets[E] unread)
 *   offsets  [E + 1]           int32  in   (from moe_permute)
 *   x        [T, d]            dtype  in   (read only if E_shared > 0)
 *   w1, w3   [E, F, d]; w2 [E, d, F]              dtype in
 *   ws1, ws3 [E_shared, F, d]; ws2 [E_shared, d, F] dtype in (NULL if
 *                                                  E_shared == 0)
 *   y_perm   [T * k, d]        dtype  out  row r = Expert(x_perm[r]) for
 *                                          r < offsets[E]; others unwritten
 *   y_shared [E_shared, T, d]  dtype  out  (NULL if E_shared == 0)
 * The SiLU-gated intermediate is kept in ws, rounded to dtype.
 */
int moe_expert_ffn(int64_t T, int64_t d_model, int32_t E, int32_t E_shared,
                   int32_t k, int64_t d_ff, int32_t dtype, const void* x_perm,
                   const int32_t* offsets, const void* x, const void* w1,
                   const void* w3, const void* w2, const void* ws1,
                   const void* ws3, const void* ws2, void* y_perm,
                   void* y_shared, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn without a workspace argument and without allocating, for
 * callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * intermediate H and the tile table live in a fixed 32 MiB device array
 * that the library holds on every GPU it runs on (one copy per device,
 * from the device's first call until the process ends).  The call
 * allocates and frees nothing.
 *   Arguments and outputs: as for moe_expert_ffn, without ws / ws_bytes.
 *   Limit: the shape's scratch (tile table + H rows (T*k + E_shared*T) x F
 *   in dtype, plus 64 MiB of split-K partials on the large-tile path that
 *   prefill-sized segments take) must fit in 32 MiB, else MOE_EWORKSPACE
 *   and nothing is launched.  Decode-shaped calls fit: the DeepSeek-V3
 *   step (T = 64, k = 8, one shared expert, F = 2048) needs 2.4 MB.
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents: calls that overlap on one GPU (two streams, or two
 *   threads) race; serialise them.  Results equal moe_expert_ffn's.
 */
int moe_expert_ffn_noalloc(int64_t T, int64_t d_model, int32_t E,
                           int32_t E_shared, int32_t k, int64_t d_ff,
                           int32_t dtype, const void* x_perm,
                           const int32_t* offsets, const void* x,
                           const void* w1, const void* w3, const void* w2,
                           const void* ws1, const void* ws3, const void* ws2,
                           void* y_perm, void* y_shared, void* stream);

/*
 * The forward of a training step ("CMU 11-868 Lecture 17" 5.2, the SwiGLU
 * expert, whose backward needs A = X W1^T and B = X W3^T): moe_expert_ffn
 * on the large grouped tiles for any shape, bf16 only, that also writes
 *   ab [T*k + E_shared*T, 2F] bf16 out: row r holds A (columns 0..F-1) and
 *     B (F..2F-1) of H row r (kept routed rows 0..R-1, then each shared
 *     expert's T rows at T*k + s*T); other routed rows unwritten.
 * y_perm and y_shared are bit-identical to moe_expert_ffn's whenever that
 * call takes the large tiles (T*k >= 64 E).  Same workspace; the caller owns
 * ab and hands it to moe_expert_ffn_backward.
 */
int moe_expert_ffn_train(int64_t T, int64_t d_model, int32_t E, int32_t E_shared,
                         int32_t k, int64_t d_ff, int32_t dtype, const void* x_perm,
                         const int32_t* offsets, const void* x, const void* w1,
                         const void* w3, const void* w2, const void* ws1, const void* ws3,
                         const void* ws2, void* y_perm, void* y_shared, void* ab, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * FP8 expert weights (the pages name FP8 expert storage, "CMU 11-868
 * Lecture 17" section 1.4, without an encoding; this library uses OCP FP8
 * E4M3 codes with one fp32 scale per stored weight row):
 *   s_r = max_i |w[r][i]| / 448   (fp32, correctly rounded; 1 for a zero row)
 *   codes[r][i] = E4M3 round-to-nearest-even of fp32(w[r][i] / s_r),
 *                 magnitudes clamped to 448
 *   the weight used is s_r * E4M3(codes[r][i])
 *   w      [rows, cols] dtype in (bf16 or fp32)
 *   codes  [rows, cols] uint8 out;  scales [rows] fp32 out
 * Quantise w1, w3 as [E*F, d] (scales [E, F]) and w2 as [E*d, F] (scales
 * [E, d]).  Rows must start 16-byte aligned for moe_expert_ffn_fp8, i.e.
 * cols a multiple of 16 (d and F are multiples of 64).
 */
int moe_quantize_fp8(int64_t rows, int64_t cols, int32_t dtype, const void* w,
                     uint8_t* codes, float* scales, void* stream);

/*
 * moe_expert_ffn with FP8 expert weights, for decode steps (T <= 64, so
 * every segment has at most 64 rows and is weight-streamed): each weight
 * byte is read once, half the bytes of bf16 weights.  Activations, H and
 * outputs are bf16, accumulation fp32:
 *   H = SiLU(s1 * (X q1^T)) (*) (s3 * (X q3^T)),  Y = s2 * (H q2^T)
 * with the row scales applied to the summed dot products.
 *   w1, w3 [E, F, d] uint8; s1, s3 [E, F] fp32; w2 [E, d, F] uint8;
 *   s2 [E, d] fp32; ws1, ws3, ws2 / ss1, ss3, ss2: the shared experts'
 *   (NULL if E_shared == 0); the other arguments as for moe_expert_ffn.
 * Returns MOE_EUNSUPPORTED for T > 64.
 */
int moe_expert_ffn_fp8(int64_t T, int64_t d_model, int32_t E, int32_t E_shared,
                       int32_t k, int64_t d_ff, const void* x_perm,
                       const int32_t* offsets, const void* x, const uint8_t* w1,
                       const uint8_t* w3, const uint8_t* w2, const float* s1,
                       const float* s3, const float* s2, const uint8_t* ws1,
                       const uint8_t* ws3, const uint8_t* ws2, const float* ss1,
                       const float* ss3, const float* ss2, void* y_perm,
                       void* y_shared, void* ws, size_t ws_bytes, void* stream);

/*
 * Weighted combine back to token order, "CMU 11-868 Lecture 17" section 2.2
 * (add back with the weights) and "MoE routing math" section 2.2 (shared
 * experts with weight 1):
 *   y[t] = sum_s y_shared[s][t] + sum_{j : row_of_pair[t][j] >= 0}
 *          topk_w[t][j] * y_perm[row_of_pair[t][j]]
 * A dropped pair adds nothing; the surviving weights are not renormalised.
 * Summation in fp32: shared experts first, then j = 0..k-1.  1 <= k <= 256
 * (expert choice passes k = E).
 *   y_perm [T*k, d] dtype in; y_shared [E_shared, T, d] dtype in (NULL if
 *   E_shared == 0); row_of_pair [T, k] int32 in; topk_w [T, k] fp32 in;
 *   y [T, d] dtype out.
 */
int moe_combine(int64_t T, int64_t d_model, int32_t E_shared, int32_t k,
                int32_t dtype, const void* y_perm, const void* y_shared,
                const int32_t* row_of_pair, const float* topk_w, void* y,
                void* stream);

/*
 * Load-balance statistics, "MoE routing math" sections 3.2 and 4.3, and the
 * router z-loss ("MoE deep dive" section 3.2), unscaled (alpha = beta = 1):
 *   f[i] = counts[i] / T   (before the drop, so sum_i f_i = k)
 *   P[i] = (1/T) sum_t softmax(logits[t])[i]
 *   scalars[0] = L_balance = E * sum_i f_i * P_i
 *   scalars[1] = z_loss    = (1/T) sum_t (logsumexp_i logits[t][i])^2
 *   scalars[2] = drop_rate = sum_i max(0, counts[i] - cap) / (T * k)
 * with cap = moe_capacity(T, E, k, CF).  Sums run in a fixed order (the
 * result is deterministic) and in fp64.
 *   logits [T, E] fp32 in; counts [E] int32 in; f, P [E] fp32 out;
 *   scalars [3] fp64 out (device memory).  Needs ws.
 */
int moe_aux_stats(int64_t T, int32_t E, int32_t k, double CF,
                  const float* logits, const int32_t* counts, float* f,
                  float* P, double* scalars, void* ws, size_t ws_bytes,
                  void* stream);

/*
 * Backward pass of the layer (bf16).  With an output
 * gradient dy and the loss L = sum(dy * y) + alpha * L_balance + beta * z
 * (the statistics of moe_aux_stats):
 *   combine ("CMU 11-868 Lecture 17" 2.2; "MoE routing math" 2.2):
 *     dO_tj = p~_tj dy_t on the row of each kept pair; dp~_tj = <dy_t, o_tj>
 *     (0 for a dropped pair); every shared expert's output gradient is dy;
 *   experts (the SwiGLU chain rule, "CMU 11-868 Lecture 17" 5.2):
 *     dH = dO W2, dA = dH (*) B (*) SiLU'(A), dB = dH (*) SiLU(A),
 *     dX = dA W1 + dB W3, dW1 = dA^T X, dW3 = dB^T X, dW2 = dO^T H;
 *   router ("MoE routing math" 2.1, 3.4; "Mixture of Experts architecture"
 *   router_z_loss): p~_t is the softmax of the selected logits, the
 *   balance loss reaches g only through P_i (f_i are counts), and
 *     dg = p~ (dp~ - <p~, dp~>) + p (*) (c - <p, c>) + 2 beta lse p / T,
 *     c_i = alpha E f_i / T;   dW_gate = x^T dg;
 *     dx_t = sum_s dX_shared[s][t] + sum_j dX_perm[row(t, j)] + dg_t W_gate^T.
 * The calls take the forward's saved tensors (x, logits, topk_idx, topk_w,
 * counts, offsets, row_of_pair, x_perm, y_perm) and one workspace of
 * moe_backward_workspace_size() bytes; weight gradients are fp32.
 */
int moe_backward_workspace_size(int64_t T, int64_t d_model, int32_t E,
                                int32_t E_shared, int32_t k, int64_t d_ff,
                                int32_t dtype, size_t* bytes);

/*
 *   dy [T, d] bf16 in; y_perm [T*k, d] bf16 in (moe_expert_ffn's output);
 *   row_of_pair, topk_w [T, k] in;
 *   dy_perm [T*k + E_shared*T, d] bf16 out: rows of kept pairs = p~ dy_t,
 *     rows T*k + s*T + t = dy_t (shared experts); other rows unwritten;
 *   dtopk_w [T, k] fp32 out.
 */
int moe_combine_backward(int64_t T, int64_t d_model, int32_t E_shared, int32_t k,
                         int32_t dtype, const void* dy, const void* y_perm,
                         const int32_t* row_of_pair, const float* topk_w,
                         void* dy_perm, float* dtopk_w, void* stream);

/*
 *   x_perm, offsets, x, w1, w3, w2, ws1, ws3, ws2: as for moe_expert_ffn;
 *   dy_perm from moe_combine_backward;
 *   dx_perm [T*k, d] bf16 out (rows of kept pairs); dx_shared [E_shared, T, d]
 *   bf16 out (NULL if E_shared == 0);
 *   dw1, dw3 [E, F, d], dw2 [E, d, F] fp32 out (zero for an expert with no
 *   rows); dws1, dws3, dws2 the shared experts' (NULL if E_shared == 0);
 *   ab: the pre-activations moe_expert_ffn_train kept for this forward, or
 *   NULL, in which case A = X W1^T and B = X W3^T are recomputed (one more
 *   grouped GEMM; the gradients are the same bits either way).
 */
int moe_expert_ffn_backward(int64_t T, int64_t d_model, int32_t E, int32_t E_shared,
                            int32_t k, int64_t d_ff, int32_t dtype,
                            const void* x_perm, const int32_t* offsets,
                            const void* x, const void* w1, const void* w3,
                            const void* w2, const void* ws1, const void* ws3,
                            const void* ws2, const void* dy_perm, void* dx_perm,
                            void* dx_shared, float* dw1, float* dw3, float* dw2,
                            float* dws1, float* dws3, float* dws2, const void* ab,
                            void* ws, size_t ws_bytes, void* stream);

/*
 *   x [T, d], w_gate [d, E] bf16 in; logits [T, E], topk_w, dtopk_w [T, k]
 *   fp32 in; topk_idx, row_of_pair [T, k], counts [E] int32 in;
 *   dx_perm, dx_shared from moe_expert_ffn_backward; alpha, beta: the loss
 *   weights of L_balance and z;
 *   dx [T, d] bf16 out; dw_gate [d, E] fp32 out.
 */
int moe_route_backward(int64_t T, int64_t d_model, int32_t E, int32_t E_shared,
                       int32_t k, int32_t dtype, const void* x, const void* w_gate,
                       const float* logits, const int32_t* topk_idx,
                       const float* topk_w, const float* dtopk_w,
                       const int32_t* counts, const int32_t* row_of_pair,
                       const void* dx_perm, const void* dx_shared, float alpha,
                       float beta, void* dx, float* dw_gate, void* ws,
                       size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
