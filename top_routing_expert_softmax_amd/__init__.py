"""MI355X (gfx950) forward pass of one softmax-top-k MoE layer.

A thin ctypes binding over libmoe.so (include/moe.h).  Every step of the
layer runs in the library's HIP kernels; this module only marshals torch
tensors (device memory and the current stream) into the C calls, with the
same names.  There is no fallback: if the library is missing or cannot be
loaded, every call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_F32 = 0
MOE_BF16 = 1

# Symbols declared in include/moe.h.
EXPORTS = ("moe_strerror", "moe_last_error", "moe_capacity", "moe_workspace_size",
           "moe_route", "moe_route_v3", "moe_update_bias", "moe_ec_capacity", "moe_route_ec",
           "moe_permute_ec", "moe_quantize_fp8", "moe_expert_ffn_fp8", "moe_permute",
           "moe_expert_ffn", "moe_expert_ffn_noalloc", "moe_expert_ffn_train", "moe_combine",
           "moe_aux_stats",
           "moe_backward_workspace_size",
           "moe_combine_backward", "moe_expert_ffn_backward", "moe_route_backward")

_lib = None


class MoEError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib():
    """Load libmoe.so once (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} not found: build it with "
            "`python -m top_routing_expert_softmax_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, f64, vp, sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                             ctypes.c_void_p, ctypes.c_size_t)
    L.moe_strerror.restype = ctypes.c_char_p
    L.moe_strerror.argtypes = [ctypes.c_int]
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_capacity.restype = ctypes.c_int
    L.moe_capacity.argtypes = [i64, i32, i32, f64, ctypes.POINTER(i64)]
    L.moe_workspace_size.restype = ctypes.c_int
    L.moe_workspace_size.argtypes = [i64, i64, i32, i32, i32, i64, i32, ctypes.POINTER(sz)]
    L.moe_route.restype = ctypes.c_int
    L.moe_route.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    f32 = ctypes.c_float
    L.moe_route_v3.restype = ctypes.c_int
    L.moe_route_v3.argtypes = [i64, i64, i32, i32, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp,
                               vp, sz, vp]
    L.moe_update_bias.restype = ctypes.c_int
    L.moe_update_bias.argtypes = [i64, i32, i32, f32, vp, vp, vp]
    L.moe_ec_capacity.restype = ctypes.c_int
    L.moe_ec_capacity.argtypes = [i64, i32, f64, ctypes.POINTER(i64)]
    L.moe_route_ec.restype = ctypes.c_int
    L.moe_route_ec.argtypes = [i64, i64, i32, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_permute_ec.restype = ctypes.c_int
    L.moe_permute_ec.argtypes = [i64, i64, i32, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_quantize_fp8.restype = ctypes.c_int
    L.moe_quantize_fp8.argtypes = [i64, i64, i32, vp, vp, vp, vp]
    L.moe_expert_ffn_fp8.restype = ctypes.c_int
    L.moe_expert_ffn_fp8.argtypes = [i64, i64, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp,
                                     vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_backward_workspace_size.restype = ctypes.c_int
    L.moe_backward_workspace_size.argtypes = [i64, i64, i32, i32, i32, i64, i32,
                                              ctypes.POINTER(sz)]
    L.moe_combine_backward.restype = ctypes.c_int
    L.moe_combine_backward.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.moe_expert_ffn_backward.restype = ctypes.c_int
    L.moe_expert_ffn_backward.argtypes = [i64, i64, i32, i32, i32, i64, i32] + [vp] * 20 + \
        [sz, vp]
    L.moe_route_backward.restype = ctypes.c_int
    L.moe_route_backward.argtypes = [i64, i64, i32, i32, i32, i32] + [vp] * 10 + [f32, f32] + \
        [vp, vp, vp, sz, vp]
    L.moe_permute.restype = ctypes.c_int
    L.moe_permute.argtypes = [i64, i64, i32, i32, f64, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                              vp, sz, vp]
    L.moe_expert_ffn.restype = ctypes.c_int
    L.moe_expert_ffn.argtypes = [i64, i64, i32, i32, i32, i64, i32, vp, vp, vp, vp, vp, vp,
                                 vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_ffn_noalloc.restype = ctypes.c_int
    L.moe_expert_ffn_noalloc.argtypes = [i64, i64, i32, i32, i32, i64, i32] + [vp] * 12
    L.moe_expert_ffn_train.restype = ctypes.c_int
    L.moe_expert_ffn_train.argtypes = [i64, i64, i32, i32, i32, i64, i32] + [vp] * 13 + \
        [sz, vp]
    L.moe_combine.restype = ctypes.c_int
    L.moe_combine.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    L.moe_aux_stats.restype = ctypes.c_int
    L.moe_aux_stats.argtypes = [i64, i32, i32, f64, vp, vp, vp, vp, vp, vp, sz, vp]
    _lib = L
    return L


def _check(fn, status):
    if status != MOE_OK:
        L = lib()
        raise MoEError(fn, status, L.moe_last_error().decode() or
                       L.moe_strerror(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------ entry points --

def moe_capacity(T, E, k, CF):
    """cap = min(T, ceil(CF*T*k/E)); CF None or <= 0 means no limit."""
    cap = ctypes.c_int64()
    _check("moe_capacity", lib().moe_capacity(T, E, k, 0.0 if CF is None else float(CF),
                                              ctypes.byref(cap)))
    return cap.value


def moe_workspace_size(T, d_model, E, E_shared, k, d_ff, dtype):
    n = ctypes.c_size_t()
    code = dtype if isinstance(dtype, int) else (MOE_BF16 if dtype == torch.bfloat16 else MOE_F32)
    _check("moe_workspace_size", lib().moe_workspace_size(T, d_model, E, E_shared, k, d_ff,
                                                          code, ctypes.byref(n)))
    return n.value


def moe_route(x, w_gate, k, logits, topk_idx, topk_w, ws, stream=None):
    T, d = x.shape
    E = w_gate.shape[1]
    _check("moe_route", lib().moe_route(T, d, E, k, _dtype_code(x), _ptr(x), _ptr(w_gate),
                                        _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(ws),
                                        0 if ws is None else ws.numel() * ws.element_size(),
                                        _stream(stream)))


def moe_route_v3(x, w_gate, bias, k, n_groups, topk_groups, route_scale, logits, topk_idx,
                 topk_w, ws, stream=None):
    T, d = x.shape
    E = w_gate.shape[1]
    _check("moe_route_v3", lib().moe_route_v3(
        T, d, E, k, n_groups, topk_groups, float(route_scale), _dtype_code(x), _ptr(x),
        _ptr(w_gate), _ptr(bias), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_update_bias(T, k, gamma, counts, bias, stream=None):
    E = bias.shape[0]
    _check("moe_update_bias", lib().moe_update_bias(T, E, k, float(gamma), _ptr(counts),
                                                    _ptr(bias), _stream(stream)))


def moe_ec_capacity(T, E, CF):
    """Expert choice: tokens per expert, min(T, floor((T // E) * CF))."""
    cap = ctypes.c_int64()
    _check("moe_ec_capacity", lib().moe_ec_capacity(T, E, float(CF), ctypes.byref(cap)))
    return cap.value


def moe_route_ec(x, w_gate, cap, logits, ec_token, ec_w, ws, stream=None):
    T, d = x.shape
    E = w_gate.shape[1]
    _check("moe_route_ec", lib().moe_route_ec(
        T, d, E, cap, _dtype_code(x), _ptr(x), _ptr(w_gate), _ptr(logits), _ptr(ec_token),
        _ptr(ec_w), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_permute_ec(ec_token, ec_w, x, offsets, row_of_te, w_te, x_perm, stream=None):
    E, cap = ec_token.shape
    T, d = x.shape
    _check("moe_permute_ec", lib().moe_permute_ec(
        T, d, E, cap, _dtype_code(x), _ptr(ec_token), _ptr(ec_w), _ptr(x), _ptr(offsets),
        _ptr(row_of_te), _ptr(w_te), _ptr(x_perm), _stream(stream)))


def ec_ffn_k(T, E, cap):
    """The k to pass moe_expert_ffn / moe_workspace_size for expert choice:
    its row bound T * k must cover the E * cap rows."""
    return max(1, -(-(E * cap) // T))


def moe_quantize_fp8(w, codes, scales, stream=None):
    """Per-row FP8 E4M3 codes and fp32 scales of a [rows, cols] weight
    tensor (any leading dims are flattened into rows)."""
    cols = w.shape[-1]
    rows = w.numel() // cols
    _check("moe_quantize_fp8", lib().moe_quantize_fp8(rows, cols, _dtype_code(w), _ptr(w),
                                                      _ptr(codes), _ptr(scales), _stream(stream)))


def moe_expert_ffn_fp8(T, k, x_perm, offsets, x, q1, q3, q2, s1, s3, s2, y_perm, ws,
                       sq1=None, sq3=None, sq2=None, ss1=None, ss3=None, ss2=None, y_shared=None,
                       stream=None):
    E, F, d = q1.shape
    Es = 0 if sq1 is None else sq1.shape[0]
    _check("moe_expert_ffn_fp8", lib().moe_expert_ffn_fp8(
        T, d, E, Es, k, F, _ptr(x_perm), _ptr(offsets), _ptr(x), _ptr(q1), _ptr(q3), _ptr(q2),
        _ptr(s1), _ptr(s3), _ptr(s2), _ptr(sq1), _ptr(sq3), _ptr(sq2), _ptr(ss1), _ptr(ss3),
        _ptr(ss2), _ptr(y_perm), _ptr(y_shared), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def moe_permute(topk_idx, x, E, CF, counts, offsets, token_of_row, row_of_pair, drop_mask,
                x_perm, ws, stream=None):
    T, k = topk_idx.shape
    d = x.shape[1]
    _check("moe_permute", lib().moe_permute(
        T, d, E, k, 0.0 if CF is None else float(CF), _dtype_code(x), _ptr(topk_idx),
        _ptr(x), _ptr(counts), _ptr(offsets), _ptr(token_of_row), _ptr(row_of_pair),
        _ptr(drop_mask), _ptr(x_perm), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def moe_expert_ffn(T, k, x_perm, offsets, x, w1, w3, w2, ws1, ws3, ws2, y_perm, y_shared,
                   ws, stream=None):
    E, F, d = w1.shape
    Es = 0 if ws1 is None else ws1.shape[0]
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        T, d, E, Es, k, F, _dtype_code(x_perm), _ptr(x_perm), _ptr(offsets), _ptr(x),
        _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(y_perm),
        _ptr(y_shared), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_expert_ffn_noalloc(T, k, x_perm, offsets, x, w1, w3, w2, ws1, ws3, ws2, y_perm,
                           y_shared, stream=None):
    """moe_expert_ffn on the library's fixed device scratch (no workspace,
    no allocation); shapes whose scratch exceeds it raise MoEError."""
    E, F, d = w1.shape
    Es = 0 if ws1 is None else ws1.shape[0]
    _check("moe_expert_ffn_noalloc", lib().moe_expert_ffn_noalloc(
        T, d, E, Es, k, F, _dtype_code(x_perm), _ptr(x_perm), _ptr(offsets), _ptr(x),
        _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(y_perm),
        _ptr(y_shared), _stream(stream)))


def moe_expert_ffn_train(T, k, x_perm, offsets, x, w1, w3, w2, ws1, ws3, ws2, y_perm, y_shared,
                         ab, ws, stream=None):
    E, F, d = w1.shape
    Es = 0 if ws1 is None else ws1.shape[0]
    _check("moe_expert_ffn_train", lib().moe_expert_ffn_train(
        T, d, E, Es, k, F, _dtype_code(x_perm), _ptr(x_perm), _ptr(offsets), _ptr(x),
        _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(y_perm),
        _ptr(y_shared), _ptr(ab), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_combine(y_perm, y_shared, row_of_pair, topk_w, y, stream=None):
    T, k = row_of_pair.shape
    d = y.shape[1]
    Es = 0 if y_shared is None else y_shared.shape[0]
    _check("moe_combine", lib().moe_combine(
        T, d, Es, k, _dtype_code(y), _ptr(y_perm), _ptr(y_shared), _ptr(row_of_pair),
        _ptr(topk_w), _ptr(y), _stream(stream)))


def moe_aux_stats(logits, counts, k, CF, f, P, scalars, ws, stream=None):
    T, E = logits.shape
    _check("moe_aux_stats", lib().moe_aux_stats(
        T, E, k, 0.0 if CF is None else float(CF), _ptr(logits), _ptr(counts), _ptr(f),
        _ptr(P), _ptr(scalars), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_backward_workspace_size(T, d_model, E, E_shared, k, d_ff):
    n = ctypes.c_size_t()
    _check("moe_backward_workspace_size", lib().moe_backward_workspace_size(
        T, d_model, E, E_shared, k, d_ff, MOE_BF16, ctypes.byref(n)))
    return n.value


def moe_combine_backward(dy, y_perm, row_of_pair, topk_w, dy_perm, dtopk_w, E_shared=0,
                         stream=None):
    T, d = dy.shape
    k = row_of_pair.shape[1]
    _check("moe_combine_backward", lib().moe_combine_backward(
        T, d, E_shared, k, _dtype_code(dy), _ptr(dy), _ptr(y_perm), _ptr(row_of_pair),
        _ptr(topk_w), _ptr(dy_perm), _ptr(dtopk_w), _stream(stream)))


def moe_expert_ffn_backward(T, k, x_perm, offsets, x, w1, w3, w2, dy_perm, dx_perm, dw1, dw3,
                            dw2, ws, ws1=None, ws3=None, ws2=None, dx_shared=None, dws1=None,
                            dws3=None, dws2=None, stream=None, ab=None):
    E, F, d = w1.shape
    Es = 0 if ws1 is None else ws1.shape[0]
    _check("moe_expert_ffn_backward", lib().moe_expert_ffn_backward(
        T, d, E, Es, k, F, _dtype_code(x_perm), _ptr(x_perm), _ptr(offsets), _ptr(x), _ptr(w1),
        _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(dy_perm), _ptr(dx_perm),
        _ptr(dx_shared), _ptr(dw1), _ptr(dw3), _ptr(dw2), _ptr(dws1), _ptr(dws3), _ptr(dws2),
        _ptr(ab), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_route_backward(x, w_gate, logits, topk_idx, topk_w, dtopk_w, counts, row_of_pair,
                       dx_perm, dx_shared, alpha, beta, dx, dw_gate, ws, E_shared=0,
                       stream=None):
    T, d = x.shape
    E = w_gate.shape[1]
    k = topk_idx.shape[1]
    _check("moe_route_backward", lib().moe_route_backward(
        T, d, E, E_shared, k, _dtype_code(x), _ptr(x), _ptr(w_gate), _ptr(logits),
        _ptr(topk_idx), _ptr(topk_w), _ptr(dtopk_w), _ptr(counts), _ptr(row_of_pair),
        _ptr(dx_perm), _ptr(dx_shared), float(alpha), float(beta), _ptr(dx), _ptr(dw_gate),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def layer_backward(x, w_gate, w1, w3, w2, k, dy, alpha, beta, fwd, ws1=None, ws3=None,
                   ws2=None, ws=None, stream=None):
    """Backward of a layer_forward() run (its buffers `fwd`): returns dx,
    dw_gate, (dw1, dw3, dw2) and the shared experts' (or None).  Uses the
    pre-activations the forward kept (save_ab=True), else recomputes them."""
    T, d = x.shape
    E, F, _ = w1.shape
    Es = 0 if ws1 is None else ws1.shape[0]
    dev = x.device
    if ws is None:
        ws = torch.empty(moe_backward_workspace_size(T, d, E, Es, k, F), dtype=torch.uint8,
                         device=dev)
    dy_perm = torch.empty((T * k + Es * T, d), dtype=x.dtype, device=dev)
    dtopk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    dx_perm = torch.empty((T * k, d), dtype=x.dtype, device=dev)
    dx_shared = torch.empty((Es, T, d), dtype=x.dtype, device=dev) if Es else None
    dw = [torch.empty(w.shape, dtype=torch.float32, device=dev) for w in (w1, w3, w2)]
    dws = ([torch.empty(w.shape, dtype=torch.float32, device=dev) for w in (ws1, ws3, ws2)]
           if Es else [None, None, None])
    dx = torch.empty_like(x)
    dw_gate = torch.empty((d, E), dtype=torch.float32, device=dev)
    moe_combine_backward(dy, fwd.y_perm, fwd.row_of_pair, fwd.topk_w, dy_perm, dtopk_w, Es,
                         stream)
    moe_expert_ffn_backward(T, k, fwd.x_perm, fwd.offsets, x, w1, w3, w2, dy_perm, dx_perm,
                            dw[0], dw[1], dw[2], ws, ws1, ws3, ws2, dx_shared, dws[0], dws[1],
                            dws[2], stream, ab=getattr(fwd, "ab", None))
    moe_route_backward(x, w_gate, fwd.logits, fwd.topk_idx, fwd.topk_w, dtopk_w, fwd.counts,
                       fwd.row_of_pair, dx_perm, dx_shared, alpha, beta, dx, dw_gate, ws, Es,
                       stream)
    return dx, dw_gate, tuple(dw), (tuple(dws) if Es else None)


# ------------------------------------------------------ whole-layer helper --

class MoELayerBuffers:
    """Device buffers for one layer shape, allocated once (torch allocator)."""

    def __init__(self, T, d_model, E, E_shared, k, d_ff, dtype, device="cuda"):
        dev = torch.device(device)
        self.T, self.d, self.E, self.Es, self.k, self.F = T, d_model, E, E_shared, k, d_ff
        self.dtype = dtype
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.token_of_row = torch.empty(T * k, dtype=torch.int32, device=dev)
        self.row_of_pair = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.drop_mask = torch.empty((T, k), dtype=torch.uint8, device=dev)
        self.x_perm = torch.empty((T * k, d_model), dtype=dtype, device=dev)
        self.y_perm = torch.empty((T * k, d_model), dtype=dtype, device=dev)
        self.y_shared = (torch.empty((E_shared, T, d_model), dtype=dtype, device=dev)
                         if E_shared else None)
        self.y = torch.empty((T, d_model), dtype=dtype, device=dev)
        self.f = torch.empty(E, dtype=torch.float32, device=dev)
        self.P = torch.empty(E, dtype=torch.float32, device=dev)
        self.scalars = torch.empty(3, dtype=torch.float64, device=dev)
        nbytes = moe_workspace_size(T, d_model, E, E_shared, k, d_ff, dtype)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.ab = None          # pre-activations, when a training forward keeps them


def layer_forward(x, w_gate, w1, w3, w2, k, CF, ws1=None, ws3=None, ws2=None, bufs=None,
                  stream=None, save_ab=False):
    """Run the five entry points in order on one stream; returns the buffers.
    save_ab: run moe_expert_ffn_train and keep the pre-activations in
    bufs.ab for layer_backward."""
    T, d = x.shape
    E, F, _ = w1.shape
    Es = 0 if ws1 is None else ws1.shape[0]
    if bufs is None:
        bufs = MoELayerBuffers(T, d, E, Es, k, F, x.dtype, device=x.device)
    b = bufs
    moe_route(x, w_gate, k, b.logits, b.topk_idx, b.topk_w, b.ws, stream)
    moe_permute(b.topk_idx, x, E, CF, b.counts, b.offsets, b.token_of_row, b.row_of_pair,
                b.drop_mask, b.x_perm, b.ws, stream)
    if save_ab:
        if b.ab is None:
            b.ab = torch.empty((T * k + Es * T, 2 * F), dtype=x.dtype, device=x.device)
        moe_expert_ffn_train(T, k, b.x_perm, b.offsets, x, w1, w3, w2, ws1, ws3, ws2, b.y_perm,
                             b.y_shared, b.ab, b.ws, stream)
    else:
        b.ab = None
        moe_expert_ffn(T, k, b.x_perm, b.offsets, x, w1, w3, w2, ws1, ws3, ws2, b.y_perm,
                       b.y_shared, b.ws, stream)
    moe_combine(b.y_perm, b.y_shared, b.row_of_pair, b.topk_w, b.y, stream)
    moe_aux_stats(b.logits, b.counts, k, CF, b.f, b.P, b.scalars, b.ws, stream)
    return b
