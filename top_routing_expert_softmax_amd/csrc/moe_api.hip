// C ABI of the MoE-layer forward (include/moe.h): argument checks, exact
// capacity, workspace sizing and error reporting around the launchers.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace {

thread_local char g_msg[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_msg[0] = '\0';
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, ...)                          \
  do {                                              \
    if (!(cond)) return fail(MOE_EINVAL, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p)                                                         \
  do {                                                                         \
    if ((p) == nullptr) return fail(MOE_EINVAL, "%s is NULL", #p);              \
    if (!aligned16(p)) return fail(MOE_EINVAL, "%s is not 16-byte aligned", #p); \
  } while (0)

int check_common(int64_t T, int32_t E, int32_t k) {
  REQUIRE(T >= 1, "T must be >= 1 (got %lld)", static_cast<long long>(T));
  REQUIRE(E >= 1 && E <= 256, "E must be in [1, 256] (got %d)", E);
  REQUIRE(k >= 1 && k <= E && k <= 64, "k must be in [1, min(E, 64)] (got k=%d, E=%d)", k, E);
  REQUIRE(T * k < (int64_t(1) << 31), "T*k must be < 2^31");
  return MOE_OK;
}

int check_dtype(int32_t dtype) {
  if (dtype != MOE_F32 && dtype != MOE_BF16)
    return fail(MOE_EUNSUPPORTED, "dtype %d has no kernel (MOE_F32=0, MOE_BF16=1)", dtype);
  return MOE_OK;
}

int check_dim(const char* name, int64_t v) {
  REQUIRE(v >= 64 && v % 64 == 0 && v < (int64_t(1) << 22),
          "%s must be a positive multiple of 64 below 2^22 (got %lld)", name,
          static_cast<long long>(v));
  return MOE_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// ceil(CF * T * k / E) on the exact value of CF, clamped to T; CF <= 0: T.
int64_t exact_capacity(int64_t T, int32_t E, int32_t k, double CF) {
  if (!(CF > 0.0)) return T;
  int ex = 0;
  const double fr = frexp(CF, &ex);                            // CF = fr * 2^ex, fr in [0.5, 1)
  const int64_t m = static_cast<int64_t>(ldexp(fr, 53));       // CF = m * 2^(ex - 53) exactly
  ex -= 53;
  __int128 num = static_cast<__int128>(m) * T * k;             // < 2^84
  int64_t c;
  if (ex >= 0) {
    if (ex >= 40) return T;                                    // the product is >= 2^40 > T
    num <<= ex;
    c = static_cast<int64_t>(std::min<__int128>((num + E - 1) / E, static_cast<__int128>(T)));
  } else {
    const int s = -ex;
    if (s >= 96) return std::min<int64_t>(T, 1);               // 0 < value < 1
    const __int128 den = static_cast<__int128>(E) << s;
    c = static_cast<int64_t>(std::min<__int128>((num + den - 1) / den, static_cast<__int128>(T)));
  }
  return std::min<int64_t>(c, T);
}

// floor((T // E) * CF) on the exact double value of CF, at most T.
int64_t ec_capacity_exact(int64_t T, int32_t E, double CF) {
  const int64_t base = T / E;
  if (base == 0 || !(CF > 0.0)) return 0;
  int ex = 0;
  const double fr = frexp(CF, &ex);
  const int64_t m = static_cast<int64_t>(ldexp(fr, 53));       // CF = m * 2^(ex - 53)
  ex -= 53;
  __int128 num = static_cast<__int128>(m) * base;              // < 2^84
  if (ex >= 0) {
    if (ex >= 40) return T;
    num <<= ex;
    return static_cast<int64_t>(std::min<__int128>(num, static_cast<__int128>(T)));
  }
  const int sh = -ex;
  if (sh >= 100) return 0;
  return static_cast<int64_t>(std::min<__int128>(num >> sh, static_cast<__int128>(T)));
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t workspace_bytes(int64_t T, int64_t d, int32_t E, int32_t Es, int32_t k, int64_t F,
                       int32_t dtype) {
  const int elem = dtype == MOE_BF16 ? 2 : 4;
  size_t b = moe::route_workspace_bytes(T, d, E);
  b = std::max(b, moe::permute_workspace_bytes(T, E));
  b = std::max(b, moe::stats_workspace_bytes(T, E));
  b = std::max(b, moe::ec_workspace_bytes(T, d, E));
  b = std::max(b, moe::ffn_workspace_bytes(T, E, Es, k, F, elem));
  return align256(b);
}

}  // namespace

// Scratch of moe_expert_ffn_noalloc: a device array that every GPU the
// library runs on holds (its own copy each) until the process ends.  Host
// code never passes the array's name to a kernel or a copy (on the host it
// is only a stand-in for the symbol): it looks up each device's address
// once, with that device current, and uses that pointer.
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// The current device's scratch address (looked up on its first use).
int current_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(MOE_EUNSUPPORTED, "moe_expert_ffn_noalloc supports device ids below %d (got %d)",
                kMaxScratchDevices, dev);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(MOE_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "success";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported dtype or shape";
    case MOE_EHIP: return "HIP error";
    case MOE_EWORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_msg; }

int moe_capacity(int64_t T, int32_t E, int32_t k, double CF, int64_t* cap) {
  if (int r = check_common(T, E, k)) return r;
  REQUIRE(cap != nullptr, "cap is NULL");
  REQUIRE(!isnan(CF) && !isinf(CF), "CF must be finite");
  *cap = exact_capacity(T, E, k, CF);
  return ok();
}

int moe_workspace_size(int64_t T, int64_t d_model, int32_t E, int32_t E_shared, int32_t k,
                       int64_t d_ff, int32_t dtype, size_t* bytes) {
  if (int r = check_common(T, E, k)) return r;
  if (int r = check_dtype(dtype)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  if (int r = check_dim("d_ff", d_ff)) return r;
  REQUIRE(E_shared >= 0 && E_shared <= 16, "E_shared must be in [0, 16]");
  REQUIRE(T * k + static_cast<int64_t>(E_shared) * T < (int64_t(1) << 31),
          "T*k + E_shared*T must be < 2^31");
  REQUIRE(bytes != nullptr, "bytes is NULL");
  *bytes = workspace_bytes(T, d_model, E, E_shared, k, d_ff, dtype);
  return ok();
}

int moe_route(int64_t T, int64_t d_model, int32_t E, int32_t k, int32_t dtype, const void* x,
              const void* w_gate, float* logits, int32_t* topk_idx, float* topk_w, void* ws,
              size_t ws_bytes, void* stream) {
  if (int r = check_common(T, E, k)) return r;
  if (int r = check_dtype(dtype)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_gate);
  REQUIRE_PTR(logits);
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(topk_w);
  const size_t need = moe::route_workspace_bytes(T, d_model, E);
  if (need > 0) {
    REQUIRE_PTR(ws);
    if (ws_bytes < need)
      return fail(MOE_EWORKSPACE, "moe_route needs %zu workspace bytes, got %zu", need, ws_bytes);
  }
  (void)hipGetLastError();
  return launched(moe::launch_route_softmax(T, d_model, E, k, dtype == MOE_BF16, x, w_gate,
                                            logits, topk_idx, topk_w, ws,
                                            static_cast<hipStream_t>(stream)),
                  "moe_route");
}

int moe_route_v3(int64_t T, int64_t d_model, int32_t E, int32_t k, int32_t n_groups,
                 int32_t topk_groups, float route_scale, int32_t dtype, const void* x,
                 const void* w_gate, const float* bias, float* logits, int32_t* topk_idx,
                 float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  if (int r = check_common(T, E, k)) return r;
  if (int r = check_dtype(dtype)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  REQUIRE(n_groups >= 1 && n_groups <= 64 && E % n_groups == 0 && E / n_groups >= 2,
          "n_groups must divide E into groups of 2 or more experts, at most 64 groups "
          "(got n_groups=%d, E=%d)", n_groups, E);
  REQUIRE(topk_groups >= 1 && topk_groups <= n_groups,
          "topk_groups must be in [1, n_groups] (got %d)", topk_groups);
  REQUIRE(static_cast<int64_t>(k) <= static_cast<int64_t>(topk_groups) * (E / n_groups),
          "k=%d exceeds the experts of the kept groups (%d)", k, topk_groups * (E / n_groups));
  REQUIRE(isfinite(route_scale) && route_scale > 0.f, "route_scale must be finite and > 0");
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_gate);
  REQUIRE_PTR(bias);
  REQUIRE_PTR(logits);
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(topk_w);
  const size_t need = moe::route_workspace_bytes(T, d_model, E);
  if (need > 0) {
    REQUIRE_PTR(ws);
    if (ws_bytes < need)
      return fail(MOE_EWORKSPACE, "moe_route_v3 needs %zu workspace bytes, got %zu", need,
                  ws_bytes);
  }
  (void)hipGetLastError();
  return launched(moe::launch_route_v3(T, d_model, E, k, n_groups, topk_groups, route_scale,
                                       dtype == MOE_BF16, x, w_gate, bias, logits, topk_idx,
                                       topk_w, ws, static_cast<hipStream_t>(stream)),
                  "moe_route_v3");
}

int moe_update_bias(int64_t T, int32_t E, int32_t k, float gamma, const int32_t* counts,
                    float* bias, void* stream) {
  if (int r = check_common(T, E, k)) return r;
  REQUIRE(isfinite(gamma), "gamma must be finite");
  REQUIRE_PTR(counts);
  REQUIRE_PTR(bias);
  (void)hipGetLastError();
  return launched(moe::launch_update_bias(T, E, k, gamma, counts, bias,
                                          static_cast<hipStream_t>(stream)),
                  "moe_update_bias");
}

int moe_ec_capacity(int64_t T, int32_t E, double CF, int64_t* cap) {
  REQUIRE(T >= 1, "T must be >= 1 (got %lld)", static_cast<long long>(T));
  REQUIRE(E >= 1 && E <= 256, "E must be in [1, 256] (got %d)", E);
  REQUIRE(cap != nullptr, "cap is NULL");
  REQUIRE(isfinite(CF) && CF >= 0.0, "CF must be finite and >= 0");
  *cap = ec_capacity_exact(T, E, CF);
  return MOE_OK;
}

static int check_ec(int64_t T, int32_t E, int64_t cap) {
  REQUIRE(T >= 1, "T must be >= 1 (got %lld)", static_cast<long long>(T));
  REQUIRE(E >= 1 && E <= 256, "E must be in [1, 256] (got %d)", E);
  REQUIRE(T * E < (int64_t(1) << 31), "T*E must be < 2^31");
  REQUIRE(cap >= 0 && cap <= T && cap <= moe::kEcMaxCap,
          "cap must be in [0, min(T, %d)] (got %lld)", moe::kEcMaxCap,
          static_cast<long long>(cap));
  return MOE_OK;
}

int moe_route_ec(int64_t T, int64_t d_model, int32_t E, int64_t cap, int32_t dtype, const void* x,
                 const void* w_gate, float* logits, int32_t* ec_token, float* ec_w, void* ws,
                 size_t ws_bytes, void* stream) {
  if (int r = check_ec(T, E, cap)) return r;
  if (int r = check_dtype(dtype)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_gate);
  REQUIRE_PTR(logits);
  if (cap > 0) {
    REQUIRE_PTR(ec_token);
    REQUIRE_PTR(ec_w);
  }
  REQUIRE_PTR(ws);
  const size_t need = moe::ec_workspace_bytes(T, d_model, E);
  if (ws_bytes < need)
    return fail(MOE_EWORKSPACE, "moe_route_ec needs %zu workspace bytes, got %zu", need, ws_bytes);
  (void)hipGetLastError();
  return launched(moe::launch_route_ec(T, d_model, E, cap, dtype == MOE_BF16, x, w_gate, logits,
                                       ec_token, ec_w, ws, static_cast<hipStream_t>(stream)),
                  "moe_route_ec");
}

int moe_permute_ec(int64_t T, int64_t d_model, int32_t E, int64_t cap, int32_t dtype,
                   const int32_t* ec_token, const float* ec_w, const void* x, int32_t* offsets,
                   int32_t* row_of_te, float* w_te, void* x_perm, void* stream) {
  if (int r = check_ec(T, E, cap)) return r;
  if (int r = check_dtype(dtype)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  if (cap > 0) {
    REQUIRE_PTR(ec_token);
    REQUIRE_PTR(ec_w);
    REQUIRE_PTR(x);
    REQUIRE_PTR(x_perm);
  }
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(row_of_te);
  REQUIRE_PTR(w_te);
  (void)hipGetLastError();
  return launched(moe::launch_permute_ec(T, d_model, E, cap, dtype == MOE_BF16, ec_token, ec_w,
                                         x, offsets, row_of_te, w_te, x_perm,
                                         static_cast<hipStream_t>(stream)),
                  "moe_permute_ec");
}

int moe_backward_workspace_size(int64_t T, int64_t d_model, int32_t E, int32_t E_shared,
                                int32_t k, int64_t d_ff, int32_t dtype, size_t* bytes) {
  if (int r = check_common(T, E, k)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  if (int r = check_dim("d_ff", d_ff)) return r;
  REQUIRE(dtype == MOE_BF16, "the backward pass runs in bf16 (dtype MOE_BF16)");
  REQUIRE(E_shared >= 0 && E_shared <= 16, "E_shared must be in [0, 16]");
  REQUIRE(bytes != nullptr, "bytes is NULL");
  *bytes = align256(std::max(moe::ffn_backward_workspace_bytes(T, d_model, E, E_shared, k, d_ff),
                             moe::route_backward_workspace_bytes(T, d_model, E)));
  return MOE_OK;
}

int moe_combine_backward(int64_t T, int64_t d_model, int32_t E_shared, int32_t k, int32_t dtype,
                         const void* dy, const void* y_perm, const int32_t* row_of_pair,
                         const float* topk_w, void* dy_perm, float* dtopk_w, void* stream) {
  REQUIRE(T >= 1, "T must be >= 1");
  REQUIRE(k >= 1 && k <= 64, "k must be in [1, 64]");
  REQUIRE(dtype == MOE_BF16, "the backward pass runs in bf16 (dtype MOE_BF16)");
  if (int r = check_dim("d_model", d_model)) return r;
  REQUIRE(E_shared >= 0 && E_shared <= 16, "E_shared must be in [0, 16]");
  REQUIRE(T * k + static_cast<int64_t>(E_shared) * T < (int64_t(1) << 31),
          "T*k + E_shared*T must be < 2^31");
  REQUIRE_PTR(dy);
  REQUIRE_PTR(y_perm);
  REQUIRE_PTR(row_of_pair);
  REQUIRE_PTR(topk_w);
  REQUIRE_PTR(dy_perm);
  REQUIRE_PTR(dtopk_w);
  (void)hipGetLastError();
  return launched(moe::launch_combine_backward(T, d_model, E_shared, k, dy, y_perm, row_of_pair,
                                               topk_w, dy_perm, dtopk_w,
                                               static_cast<hipStream_t>(stream)),
                  "moe_combine_backward");
}

int moe_expert_ffn_backward(int64_t T, int64_t d_model, int32_t E, int32_t E_shared, int32_t k,
                            int64_t d_ff, int32_t dtype, const void* x_perm,
                            const int32_t* offsets, const void* x, const void* w1,
                            const void* w3, const void* w2, const void* ws1, const void* ws3,
                            const void* ws2, const void* dy_perm, void* dx_perm, void* dx_shared,
                            float* dw1, float* dw3, float* dw2, float* dws1, float* dws3,
                            float* dws2, const void* ab, void* ws, size_t ws_bytes,
                            void* stream) {
  if (int r = check_common(T, E, k)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  if (int r = check_dim("d_ff", d_ff)) return r;
  REQUIRE(dtype == MOE_BF16, "the backward pass runs in bf16 (dtype MOE_BF16)");
  REQUIRE(E_shared >= 0 && E_shared <= 16, "E_shared must be in [0, 16]");
  REQUIRE(T * k + static_cast<int64_t>(E_shared) * T < (int64_t(1) << 31),
          "T*k + E_shared*T must be < 2^31");
  REQUIRE_PTR(x_perm);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(w1);
  REQUIRE_PTR(w3);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(dy_perm);
  REQUIRE_PTR(dx_perm);
  REQUIRE_PTR(dw1);
  REQUIRE_PTR(dw3);
  REQUIRE_PTR(dw2);
  REQUIRE_PTR(ws);
  REQUIRE(ab == nullptr || aligned16(ab), "ab is not 16-byte aligned");
  if (E_shared > 0) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(ws1);
    REQUIRE_PTR(ws3);
    REQUIRE_PTR(ws2);
    REQUIRE_PTR(dx_shared);
    REQUIRE_PTR(dws1);
    REQUIRE_PTR(dws3);
    REQUIRE_PTR(dws2);
  }
  const size_t need = moe::ffn_backward_workspace_bytes(T, d_model, E, E_shared, k, d_ff);
  if (ws_bytes < need)
    return fail(MOE_EWORKSPACE, "moe_expert_ffn_backward needs %zu workspace bytes, got %zu",
                need, ws_bytes);
  (void)hipGetLastError();
  return launched(moe::launch_expert_ffn_backward(T, d_model, E, E_shared, k, d_ff, x_perm,
                                                  offsets, x, w1, w3, w2, ws1, ws3, ws2, dy_perm,
                                                  dx_perm, dx_shared, dw1, dw3, dw2, dws1, dws3,
                                                  dws2, ab, ws, static_cast<hipStream_t>(stream)),
                  "moe_expert_ffn_backward");
}

int moe_route_backward(int64_t T, int64_t d_model, int32_t E, int32_t E_shared, int32_t k,
                       int32_t dtype, const void* x, const void* w_gate, const float* logits,
                       const int32_t* topk_idx, const float* topk_w, const float* dtopk_w,
                       const int32_t* counts, const int32_t* row_of_pair, const void* dx_perm,
                       const void* dx_shared, float alpha, float beta, void* dx, float* dw_gate,
                       void* ws, size_t ws_bytes, void* stream) {
  if (int r = check_common(T, E, k)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  REQUIRE(dtype == MOE_BF16, "the backward pass runs in bf16 (dtype MOE_BF16)");
  REQUIRE(E_shared >= 0 && E_shared <= 16, "E_shared must be in [0, 16]");
  REQUIRE(isfinite(alpha) && isfinite(beta), "alpha and beta must be finite");
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_gate);
  REQUIRE_PTR(logits);
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(topk_w);
  REQUIRE_PTR(dtopk_w);
  REQUIRE_PTR(counts);
  REQUIRE_PTR(row_of_pair);
  REQUIRE_PTR(dx_perm);
  REQUIRE_PTR(dx);
  REQUIRE_PTR(dw_gate);
  REQUIRE_PTR(ws);
  if (E_shared > 0) REQUIRE_PTR(dx_shared);
  const size_t need = moe::route_backward_workspace_bytes(T, d_model, E);
  if (ws_bytes < need)
    return fail(MOE_EWORKSPACE, "moe_route_backward needs %zu workspace bytes, got %zu", need,
                ws_bytes);
  (void)hipGetLastError();
  return launched(moe::launch_route_backward(T, d_model, E, E_shared, k, x, w_gate, logits,
                                             topk_idx, topk_w, dtopk_w, counts, row_of_pair,
                                             dx_perm, dx_shared, alpha, beta, dx, dw_gate, ws,
                                             static_cast<hipStream_t>(stream)),
                  "moe_route_backward");
}

int moe_quantize_fp8(int64_t rows, int64_t cols, int32_t dtype, const void* w, uint8_t* codes,
                     float* scales, void* stream) {
  REQUIRE(rows >= 1 && rows < (int64_t(1) << 31), "rows must be in [1, 2^31)");
  REQUIRE(cols >= 1 && cols < (int64_t(1) << 31), "cols must be in [1, 2^31)");
  if (int r = check_dtype(dtype)) return r;
  REQUIRE_PTR(w);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  (void)hipGetLastError();
  return launched(moe::launch_quantize_fp8(rows, cols, dtype == MOE_BF16, w, codes, scales,
                                           static_cast<hipStream_t>(stream)),
                  "moe_quantize_fp8");
}

int moe_expert_ffn_fp8(int64_t T, int64_t d_model, int32_t E, int32_t E_shared, int32_t k,
                       int64_t d_ff, const void* x_perm, const int32_t* offsets, const void* x,
                       const uint8_t* w1, const uint8_t* w3, const uint8_t* w2, const float* s1,
                       const float* s3, const float* s2, const uint8_t* ws1, const uint8_t* ws3,
                       const uint8_t* ws2, const float* ss1, const float* ss3, const float* ss2,
                       void* y_perm, void* y_shared, void* ws, size_t ws_bytes, void* stream) {
  if (int r = check_common(T, E, k)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  if (int r = check_dim("d_ff", d_ff)) return r;
  REQUIRE(E_shared >= 0 && E_shared <= 16, "E_shared must be in [0, 16]");
  if (T > moe::kStreamMaxRows)
    return fail(MOE_EUNSUPPORTED, "moe_expert_ffn_fp8 runs decode steps: T must be <= %d "
                "(got %lld)", moe::kStreamMaxRows, static_cast<long long>(T));
  REQUIRE_PTR(x_perm);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(w1);
  REQUIRE_PTR(w3);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(s1);
  REQUIRE_PTR(s3);
  REQUIRE_PTR(s2);
  REQUIRE_PTR(y_perm);
  REQUIRE_PTR(ws);
  if (E_shared > 0) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(ws1);
    REQUIRE_PTR(ws3);
    REQUIRE_PTR(ws2);
    REQUIRE_PTR(ss1);
    REQUIRE_PTR(ss3);
    REQUIRE_PTR(ss2);
    REQUIRE_PTR(y_shared);
  }
  const size_t need = static_cast<size_t>(T * k + static_cast<int64_t>(E_shared) * T) * d_ff * 2;
  if (ws_bytes < need)
    return fail(MOE_EWORKSPACE, "moe_expert_ffn_fp8 needs %zu workspace bytes, got %zu", need,
                ws_bytes);
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = moe::launch_ffn_stream(1, T, d_model, E, E_shared, k, d_ff, x_perm, offsets,
                                          x, w1, w3, w2, ws1, ws3, ws2, ws, y_perm, y_shared, st,
                                          s1, s3, s2, ss1, ss3, ss2);
  if (err == hipSuccess)
    err = moe::launch_ffn_stream(2, T, d_model, E, E_shared, k, d_ff, x_perm, offsets, x, w1, w3,
                                 w2, ws1, ws3, ws2, ws, y_perm, y_shared, st, s1, s3, s2, ss1,
                                 ss3, ss2);
  return launched(err, "moe_expert_ffn_fp8");
}

int moe_permute(int64_t T, int64_t d_model, int32_t E, int32_t k, double CF, int32_t dtype,
                const int32_t* topk_idx, const void* x, int32_t* counts, int32_t* offsets,
                int32_t* token_of_row, int32_t* row_of_pair, uint8_t* drop_mask, void* x_perm,
                void* ws, size_t ws_bytes, void* stream) {
  if (int r = check_common(T, E, k)) return r;
  if (int r = check_dtype(dtype)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  REQUIRE(!isnan(CF) && !isinf(CF), "CF must be finite");
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(x);
  REQUIRE_PTR(counts);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(token_of_row);
  REQUIRE_PTR(row_of_pair);
  REQUIRE_PTR(drop_mask);
  REQUIRE_PTR(x_perm);
  REQUIRE_PTR(ws);
  const size_t need = moe::permute_workspace_bytes(T, E);
  if (ws_bytes < need)
    return fail(MOE_EWORKSPACE, "moe_permute needs %zu workspace bytes, got %zu", need, ws_bytes);
  const int64_t cap = exact_capacity(T, E, k, CF);
  (void)hipGetLastError();
  return launched(moe::launch_permute(T, d_model, E, k, cap, dtype == MOE_BF16, topk_idx, x,
                                      counts, offsets, token_of_row, row_of_pair, drop_mask,
                                      x_perm, ws, static_cast<hipStream_t>(stream)),
                  "moe_permute");
}

int moe_expert_ffn(int64_t T, int64_t d_model, int32_t E, int32_t E_shared, int32_t k,
                   int64_t d_ff, int32_t dtype, const void* x_perm, const int32_t* offsets,
                   const void* x, const void* w1, const void* w3, const void* w2,
                   const void* ws1, const void* ws3, const void* ws2, void* y_perm,
                   void* y_shared, void* ws, size_t ws_bytes, void* stream) {
  if (int r = check_common(T, E, k)) return r;
  if (int r = check_dtype(dtype)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  if (int r = check_dim("d_ff", d_ff)) return r;
  REQUIRE(E_shared >= 0 && E_shared <= 16, "E_shared must be in [0, 16]");
  REQUIRE(T * k + static_cast<int64_t>(E_shared) * T < (int64_t(1) << 31),
          "T*k + E_shared*T must be < 2^31");
  REQUIRE_PTR(x_perm);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(w1);
  REQUIRE_PTR(w3);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(y_perm);
  REQUIRE_PTR(ws);
  if (E_shared > 0) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(ws1);
    REQUIRE_PTR(ws3);
    REQUIRE_PTR(ws2);
    REQUIRE_PTR(y_shared);
  }
  const size_t need = moe::ffn_workspace_bytes(T, E, E_shared, k, d_ff, dtype == MOE_BF16 ? 2 : 4);
  if (ws_bytes < need)
    return fail(MOE_EWORKSPACE, "moe_expert_ffn needs %zu workspace bytes, got %zu", need,
                ws_bytes);
  (void)hipGetLastError();
  return launched(moe::launch_expert_ffn(T, d_model, E, E_shared, k, d_ff, dtype == MOE_BF16,
                                         x_perm, offsets, x, w1, w3, w2, ws1, ws3, ws2, y_perm,
                                         y_shared, ws, static_cast<hipStream_t>(stream)),
                  "moe_expert_ffn");
}

int moe_expert_ffn_noalloc(int64_t T, int64_t d_model, int32_t E, int32_t E_shared, int32_t k,
                           int64_t d_ff, int32_t dtype, const void* x_perm,
                           const int32_t* offsets, const void* x, const void* w1, const void* w3,
                           const void* w2, const void* ws1, const void* ws3, const void* ws2,
                           void* y_perm, void* y_shared, void* stream) {
  if (int r = check_common(T, E, k)) return r;
  if (int r = check_dtype(dtype)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  if (int r = check_dim("d_ff", d_ff)) return r;
  REQUIRE(E_shared >= 0 && E_shared <= 16, "E_shared must be in [0, 16]");
  REQUIRE(T * k + static_cast<int64_t>(E_shared) * T < (int64_t(1) << 31),
          "T*k + E_shared*T must be < 2^31");
  REQUIRE_PTR(x_perm);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(w1);
  REQUIRE_PTR(w3);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(y_perm);
  if (E_shared > 0) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(ws1);
    REQUIRE_PTR(ws3);
    REQUIRE_PTR(ws2);
    REQUIRE_PTR(y_shared);
  }
  const size_t need =
      moe::ffn_workspace_used_bytes(T, E, E_shared, k, d_ff, dtype == MOE_BF16 ? 2 : 4);
  if (need > kNoallocScratchBytes)
    return fail(MOE_EWORKSPACE,
                "moe_expert_ffn_noalloc needs %zu bytes of scratch for this shape; the library "
                "holds %zu (use moe_expert_ffn with a workspace)",
                need, kNoallocScratchBytes);
  void* ws = nullptr;
  if (int r = current_scratch(&ws)) return r;
  (void)hipGetLastError();
  return launched(moe::launch_expert_ffn(T, d_model, E, E_shared, k, d_ff, dtype == MOE_BF16,
                                         x_perm, offsets, x, w1, w3, w2, ws1, ws3, ws2, y_perm,
                                         y_shared, ws, static_cast<hipStream_t>(stream)),
                  "moe_expert_ffn_noalloc");
}

int moe_expert_ffn_train(int64_t T, int64_t d_model, int32_t E, int32_t E_shared, int32_t k,
                         int64_t d_ff, int32_t dtype, const void* x_perm, const int32_t* offsets,
                         const void* x, const void* w1, const void* w3, const void* w2,
                         const void* ws1, const void* ws3, const void* ws2, void* y_perm,
                         void* y_shared, void* ab, void* ws, size_t ws_bytes, void* stream) {
  if (int r = check_common(T, E, k)) return r;
  REQUIRE(dtype == MOE_BF16, "moe_expert_ffn_train runs in bf16 (dtype MOE_BF16)");
  if (int r = check_dim("d_model", d_model)) return r;
  if (int r = check_dim("d_ff", d_ff)) return r;
  REQUIRE(E_shared >= 0 && E_shared <= 16, "E_shared must be in [0, 16]");
  REQUIRE(T * k + static_cast<int64_t>(E_shared) * T < (int64_t(1) << 31),
          "T*k + E_shared*T must be < 2^31");
  REQUIRE_PTR(x_perm);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(w1);
  REQUIRE_PTR(w3);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(y_perm);
  REQUIRE_PTR(ab);
  REQUIRE_PTR(ws);
  if (E_shared > 0) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(ws1);
    REQUIRE_PTR(ws3);
    REQUIRE_PTR(ws2);
    REQUIRE_PTR(y_shared);
  }
  const size_t need = moe::ffn_workspace_bytes(T, E, E_shared, k, d_ff, 2);
  if (ws_bytes < need)
    return fail(MOE_EWORKSPACE, "moe_expert_ffn_train needs %zu workspace bytes, got %zu", need,
                ws_bytes);
  (void)hipGetLastError();
  return launched(moe::launch_expert_ffn_train(T, d_model, E, E_shared, k, d_ff, x_perm, offsets,
                                               x, w1, w3, w2, ws1, ws3, ws2, y_perm, y_shared, ab,
                                               ws, static_cast<hipStream_t>(stream)),
                  "moe_expert_ffn_train");
}

int moe_combine(int64_t T, int64_t d_model, int32_t E_shared, int32_t k, int32_t dtype,
                const void* y_perm, const void* y_shared, const int32_t* row_of_pair,
                const float* topk_w, void* y, void* stream) {
  REQUIRE(T >= 1, "T must be >= 1");
  REQUIRE(k >= 1 && k <= 256, "k must be in [1, 256]");
  REQUIRE(T * k < (int64_t(1) << 31), "T*k must be < 2^31");
  if (int r = check_dtype(dtype)) return r;
  if (int r = check_dim("d_model", d_model)) return r;
  REQUIRE(E_shared >= 0 && E_shared <= 16, "E_shared must be in [0, 16]");
  REQUIRE_PTR(y_perm);
  REQUIRE_PTR(row_of_pair);
  REQUIRE_PTR(topk_w);
  REQUIRE_PTR(y);
  if (E_shared > 0) REQUIRE_PTR(y_shared);
  (void)hipGetLastError();
  return launched(moe::launch_combine(T, d_model, E_shared, k, dtype == MOE_BF16, y_perm,
                                      y_shared, row_of_pair, topk_w, y,
                                      static_cast<hipStream_t>(stream)),
                  "moe_combine");
}

int moe_aux_stats(int64_t T, int32_t E, int32_t k, double CF, const float* logits,
                  const int32_t* counts, float* f, float* P, double* scalars, void* ws,
                  size_t ws_bytes, void* stream) {
  if (int r = check_common(T, E, k)) return r;
  REQUIRE(!isnan(CF) && !isinf(CF), "CF must be finite");
  REQUIRE_PTR(logits);
  REQUIRE_PTR(counts);
  REQUIRE_PTR(f);
  REQUIRE_PTR(P);
  REQUIRE(scalars != nullptr && (reinterpret_cast<uintptr_t>(scalars) & 7u) == 0,
          "scalars must be a non-NULL 8-byte aligned pointer");
  REQUIRE_PTR(ws);
  const size_t need = moe::stats_workspace_bytes(T, E);
  if (ws_bytes < need)
    return fail(MOE_EWORKSPACE, "moe_aux_stats needs %zu workspace bytes, got %zu", need,
                ws_bytes);
  const int64_t cap = exact_capacity(T, E, k, CF);
  (void)hipGetLastError();
  return launched(moe::launch_aux_stats(T, E, k, cap, logits, counts, f, P, scalars, ws,
                                        static_cast<hipStream_t>(stream)),
                  "moe_aux_stats");
}

}  // extern "C"
