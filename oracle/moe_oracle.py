"""Plain, slow, fp64 CPU oracle of one MoE layer's forward pass.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the HIP product path, and it shares no
code with it.  Every function works in float64 on the exact values that the
device receives (bf16 inputs are widened, never re-rounded).

Sources, cited by page title and section:
  [RM]  "MoE routing math" (jerryiiii.gitbook.io, llm-review math dictionary)
  [SA]  "Mixture of Experts architecture: how sparse activation reshapes the
        efficiency and scale of LLMs" (x7peeps.com); its listings are named
        by their function names (moe_forward, load_balancing_loss,
        router_z_loss)
  [DD]  "MoE deep dive: routing mechanisms and load balancing" (guijiagi.com)
  [L17] "CMU 11-868 Lecture 17: Systems for Mixture-of-Experts Models"
        (semidirectx.com notes)
  [INF] "MoE inference optimisation, deep dive" (jerryiiii.gitbook.io notes)

Readings where the pages are silent or disagree:
  * top-k order: larger first; equal values go to the lower expert index.
  * capacity: ceil(CF * T * k / E) evaluated exactly on the given CF value,
    clamped to T; CF None or <= 0 means no limit (cap = T).
  * overflow: within each expert the lowest token indices are kept.
  * a dropped (token, choice) contributes zero and the surviving weights are
    not renormalised.
  * f_i is counted before the drop (sum_i f_i = k); N = T.
  * SiLU(z) = z * sigmoid(z); W1 is the gated branch, W3 the linear one.
  * DeepSeek-V3 gate: the affinity sigmoid(g) is evaluated in fp64 and
    rounded once to fp32; the bias add, the two-largest group sums and every
    comparison that picks groups and experts are fp32 (the precision of the
    kernel, so both sides take the same integer decisions); ties go to the
    lower group / expert index; the bias rule compares counts_i with the
    mean T k / E exactly.
  * expert choice: capacity = floor((T // E) * CF) as the listing writes
    it, clamped to T; each expert takes its capacity tokens with the largest
    logits (ties to the lower token); the pages give no combine weight, so a
    chosen (token, expert) pair is weighted by the router probability
    softmax(g_t)_e, not renormalised, and a token no expert chose outputs 0.
  * FP8 expert weights: the pages name FP8 storage but no encoding or scale;
    taken here: OCP FP8 E4M3 (bias 7, no infinities, largest finite 448),
    one fp32 scale per stored weight row s = max|w_row| / 448 (fp32
    division), codes = round-to-nearest-even of the fp32 quotient w / s,
    clamped to +-448; the weight the layer uses is s * decode(code).
  * backward: the loss is L = sum(dy * y) + alpha * L_balance + beta * z;
    the balance loss reaches the router through P_i only (f_i are counts);
    a dropped pair contributes nothing, but its weight stays in the
    softmax over the token's selected logits that p~ is.
"""
from fractions import Fraction
import math

import numpy as np

__all__ = [
    "router_logits", "softmax", "logsumexp", "topk_experts",
    "renormalise", "topk_softmax_weights", "route", "expert_counts",
    "capacity", "dispatch", "silu", "swiglu_expert", "combine_grouped",
    "combine_per_token", "load_balance_loss", "aux_stats", "layer_forward",
    "affinity_f32", "v3_gate", "update_bias",
    "ec_capacity", "expert_choice", "ec_dispatch", "ec_combine",
    "e4m3_decode", "e4m3_encode", "quantize_fp8_rows", "dequantize_fp8_rows",
    "silu_grad", "swiglu_expert_backward", "layer_backward", "router_logit_grad",
    "layer_backward_sampled",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- routing --

def router_logits(x, w_gate):
    """g = x . W_gate, W_gate in R^{d x E}, no bias.  [RM] section 2.1."""
    return _f64(x) @ _f64(w_gate)


def softmax(g):
    """p = softmax(g) over the E routed experts.  [RM] section 2.1."""
    g = _f64(g)
    m = g.max(axis=-1, keepdims=True)
    e = np.exp(g - m)
    return e / e.sum(axis=-1, keepdims=True)


def logsumexp(g):
    """log sum_i exp(g_i), the quantity the z-loss squares.  [SA]
    router_z_loss; [DD] section 3.2."""
    g = _f64(g)
    m = g.max(axis=-1)
    return m + np.log(np.exp(g - m[..., None]).sum(axis=-1))


def topk_experts(scores, k):
    """S = TopK(scores, k) per row: indices of the k largest, larger first,
    ties to the lower expert index.  [RM] section 2.1 (TopK over p)."""
    scores = _f64(scores)
    order = np.argsort(-scores, axis=-1, kind="stable")
    return order[..., :k].astype(np.int64)


def renormalise(p, idx):
    """p~_i = p_i / sum_{j in S} p_j for i in S.  [RM] section 2.1."""
    sel = np.take_along_axis(_f64(p), idx, axis=-1)
    return sel / sel.sum(axis=-1, keepdims=True)


def topk_softmax_weights(g, k):
    """Second form of the same weights: take the k largest logits first, then
    softmax over only those.  [SA] moe_forward steps 2-3; [DD] section 2.1
    (TopKRouter); called top-k-softmax (Mixtral) in [L17] section 6."""
    idx = topk_experts(g, k)
    return idx, softmax(np.take_along_axis(_f64(g), idx, axis=-1))


def route(x, w_gate, k):
    """Router: logits, probabilities, top-k indices, renormalised weights and
    the per-token log-sum-exp.  The top-k is taken over p as [RM] section 2.1
    writes it."""
    g = router_logits(x, w_gate)
    p = softmax(g)
    idx = topk_experts(p, k)
    w = renormalise(p, idx)
    return {"logits": g, "probs": p, "idx": idx, "weights": w,
            "lse": logsumexp(g)}


# ------------------------------------------------- DeepSeek-V3 gate (N1) --

def affinity_f32(g):
    """s = sigmoid(g), one affinity in (0, 1) per expert ([L17] section 5.3,
    first step of the V3 gate).  Evaluated in fp64 and rounded once to fp32,
    the precision in which the gate takes its decisions."""
    g = _f64(g)
    return (1.0 / (1.0 + np.exp(-g))).astype(np.float32)


def v3_gate(g, bias, k, n_groups, topk_groups, route_scale):
    """DeepSeek-V3 gate, sigmoid branch ([L17] section 5.3, with the
    selection-only bias of section 3.4), in its steps:

      1. s = sigmoid(g) per expert;
      2. biased = s + b: the balance bias enters only the choice;
      3. the E experts form n_groups contiguous groups; a group's score is
         the sum of its two largest biased scores;
      4. the topk_groups best groups are kept, the others masked out;
      5. the k largest biased scores among the kept experts are chosen;
      6. the weights are the UNBIASED affinities of the chosen experts,
         divided by their sum and multiplied by route_scale.

    Steps 2-5 are fp32 (see the module notes); step 6 is fp64.  Returns the
    chosen ids (larger biased score first, ties to the lower index), the
    weights and the intermediate arrays."""
    s = affinity_f32(g)
    T, E = s.shape
    if E % n_groups or E // n_groups < 2:
        raise ValueError("groups must split E evenly, two experts or more each")
    b = np.asarray(bias, dtype=np.float32)
    biased = s + b[None, :]                                   # fp32 + fp32
    G = E // n_groups
    ranked = -np.sort(-biased.reshape(T, n_groups, G), axis=-1)
    gscore = ranked[..., 0] + ranked[..., 1]                  # fp32 sum of the two largest
    kept = np.argsort(-gscore, axis=-1, kind="stable")[:, :topk_groups]
    in_kept = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(in_kept, kept, True, axis=-1)
    allowed = np.repeat(in_kept, G, axis=-1)
    masked = np.where(allowed, biased.astype(np.float64), -np.inf)
    idx = np.argsort(-masked, axis=-1, kind="stable")[:, :k].astype(np.int64)
    sel = np.take_along_axis(_f64(s), idx, axis=-1)
    w = sel / sel.sum(axis=-1, keepdims=True) * float(route_scale)
    return {"idx": idx, "weights": w, "affinity": s, "biased": biased,
            "group_score": gscore, "kept_groups": kept, "logits": _f64(g)}


def update_bias(counts, bias, T, k, gamma):
    """Balance-bias step of DeepSeek-V3 ([L17] section 3.4; [SA]
    update_bias): an expert loaded above the mean T k / E loses gamma, one
    below it gains gamma, one exactly at it keeps its bias.  fp32, like the
    stored bias."""
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.shape[0]
    b = np.asarray(bias, dtype=np.float32).copy()
    gam = np.float32(gamma)
    over = counts * E > T * k
    under = counts * E < T * k
    b[over] = b[over] - gam
    b[under] = b[under] + gam
    return b


# ------------------------------------------------- expert choice (N3) --

def ec_capacity(T, E, CF):
    """Tokens per expert under expert choice: T // E tokens times the
    capacity factor ([DD] section 2.2, ExpertChoiceRouter), floored (a top-k
    size is an integer), at most T."""
    c = Fraction(T // E) * Fraction(CF)
    return int(min(T, max(0, c.numerator // c.denominator)))


def expert_choice(g, cap):
    """Expert choice ([DD] section 2.2): transpose the logits so experts come
    first, and let each expert take the cap tokens with the largest logits
    (larger first, ties to the lower token index).  Weights: the router
    probability softmax(g_t)_e of each chosen pair ([RM] section 2.1's p;
    the listing leaves the weight open)."""
    g = _f64(g)
    gt = g.T
    tokens = np.argsort(-gt, axis=-1, kind="stable")[:, :cap].astype(np.int64)
    p = softmax(g)
    E = g.shape[1]
    w = np.stack([p[tokens[e], e] for e in range(E)]) if cap else np.zeros((E, 0))
    return {"logits": g, "probs": p, "tokens": tokens, "weights": w}


def ec_dispatch(tokens, weights, T):
    """Rows of the grouped layout: expert e owns rows e*cap .. e*cap+cap-1,
    row e*cap+j holding token tokens[e][j] ([L17] section 2.2, one segment
    per expert).  row_of_te[t][e] is that row or -1, w_te[t][e] its weight
    or 0."""
    E, cap = tokens.shape
    row_of_te = -np.ones((T, E), dtype=np.int64)
    w_te = np.zeros((T, E))
    for e in range(E):
        for j in range(cap):
            row_of_te[tokens[e, j], e] = e * cap + j
            w_te[tokens[e, j], e] = weights[e, j]
    return {"offsets": np.arange(E + 1, dtype=np.int64) * cap,
            "token_of_row": tokens.reshape(-1), "row_of_te": row_of_te, "w_te": w_te}


def ec_combine(x, tokens, weights, load_expert, shared_out=None):
    """y_t = sum_s Shared_s(x_t) + sum over experts e that chose t of
    w_{t,e} Expert_e(x_t); per expert, one product over its chosen rows."""
    x = _f64(x)
    y = np.zeros_like(x)
    if shared_out is not None:
        y += _f64(shared_out)
    for e in range(tokens.shape[0]):
        if tokens.shape[1] == 0:
            break
        out = swiglu_expert(x[tokens[e]], *load_expert(e))
        for j, t in enumerate(tokens[e]):
            y[t] += weights[e, j] * out[j]
    return y


# ----------------------------------------------- FP8 expert weights (N4) --

def e4m3_decode(codes):
    """Value of OCP FP8 E4M3 codes: sign bit, 4 exponent bits (bias 7), 3
    mantissa bits; exponent 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN
    (never produced here)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_encode(v):
    """Round-to-nearest-even of fp32 values to E4M3 codes, saturating at
    +-448.  Exact on the fp32 input: |v| = q * step with step = 2^(E-3) the
    grid spacing of its binade 2^E (2^-9 below 2^-6, the subnormals), so
    rint(q) (ties to even) picks the nearest grid value."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    sign = np.signbit(v)
    a = np.minimum(np.abs(v), 448.0)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))          # a = f 2^ex, f in [0.5, 1)
    step = np.ldexp(1.0, ex - 4)                        # 2^(E-3) with E = ex - 1
    val = np.rint(a / step) * step                      # nearest, ties to even
    sub = val < 2.0 ** -6
    _, ev = np.frexp(np.where(sub, 1.0, val))
    E = ev - 1
    m = np.where(sub, 0, np.rint(np.ldexp(val, -E) * 8) - 8)
    code = np.where(sub, np.rint(val * 2.0 ** 9), ((E + 7) << 3) + m).astype(np.int64)
    return np.where(sign, code | 0x80, code).astype(np.uint8)


def quantize_fp8_rows(w):
    """Per-row FP8 quantisation of a weight matrix (rows = the stored rows,
    each one output feature): s = fp32(max|w_row|) / 448 in fp32, codes =
    E4M3 RNE of fp32(w / s).  All-zero rows get s = 1.  Returns (codes,
    scales)."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=-1)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = (w / s[..., None]).astype(np.float32)
    return e4m3_encode(q), s


def dequantize_fp8_rows(codes, scales):
    """The weights the FP8 layer computes with: s * decode(code), fp64."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


# --------------------------------------------------------------- dispatch --

def expert_counts(idx, E):
    """Number of (token, choice) pairs that picked each expert, before any
    drop.  [SA] load_balancing_loss (the one-hot mask summed over tokens)."""
    return np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.int64)


def capacity(T, E, k, CF):
    """capacity = ceil(cf * k * n / E), [L17] section 2.4, with n = T tokens,
    evaluated exactly on the float value given.  A token picks an expert at
    most once, so the result is clamped to T.  CF None or <= 0: no limit."""
    if CF is None or CF <= 0:
        return int(T)
    c = Fraction(CF) * T * k / E
    return int(min(T, math.ceil(c)))


def dispatch(idx, E, cap):
    """Group (token, choice) pairs by expert in token order and drop what
    exceeds the capacity.  [L17] section 2.2 (group by expert), section 2.4
    (overflow is dropped); [RM] section 4.3 (drop rate over pairs).

    Returns slot (rank inside the expert's kept rows, -1 if dropped), the
    drop mask, kept rows per expert, offsets (exclusive scan of kept),
    row_of_pair (offsets[e] + slot, -1 if dropped) and token_of_row (the
    inverse map, -1 past the last kept row; rows run over T*k slots)."""
    idx = np.asarray(idx)
    T, k = idx.shape
    fill = [0] * E
    slot = np.full((T, k), -1, dtype=np.int64)
    drop = np.zeros((T, k), dtype=np.uint8)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if fill[e] < cap:
                slot[t, j] = fill[e]
                fill[e] += 1
            else:
                drop[t, j] = 1
    kept = np.array(fill, dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    row_of_pair = np.full((T, k), -1, dtype=np.int64)
    token_of_row = np.full(T * k, -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if not drop[t, j]:
                r = offsets[idx[t, j]] + slot[t, j]
                row_of_pair[t, j] = r
                token_of_row[r] = t
    return {"slot": slot, "drop": drop, "kept": kept, "offsets": offsets,
            "row_of_pair": row_of_pair, "token_of_row": token_of_row}


# ------------------------------------------------------------------ experts --

def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(xr, w1, w3, w2):
    """FFN(x) = (SiLU(x W1) (*) x W3) W2, [L17] section 5.2.

    Weights come in storage layout: w1, w3 [F, d] hold W1, W3 transposed and
    w2 [d, F] holds W2 transposed."""
    xr = _f64(xr)
    a = xr @ _f64(w1).T
    b = xr @ _f64(w3).T
    return (silu(a) * b) @ _f64(w2).T


def combine_grouped(x, weights, idx, disp, load_expert, E, tokens=None,
                    shared_out=None):
    """Grouped form: per expert, gather the kept rows, run the expert once on
    all of them, and add p~-weighted results back in token order.
    [L17] section 2.2 (group, one product per expert, index_add back).

    tokens restricts the output to those token indices (others are not
    computed); load_expert(e) -> (w1, w3, w2) in storage layout;
    shared_out, if given, is added first (always-on shared experts,
    [RM] section 2.2)."""
    x = _f64(x)
    T = x.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    pos = {int(t): i for i, t in enumerate(tok)}
    y = np.zeros((len(tok), x.shape[1]))
    if shared_out is not None:
        y += _f64(shared_out)
    kept = disp["drop"] == 0
    for e in range(E):
        sel = [(int(t), j) for t, j in zip(*np.nonzero((np.asarray(idx) == e) & kept))
               if int(t) in pos]
        if not sel:
            continue
        w1, w3, w2 = load_expert(e)
        rows = np.array([t for t, _ in sel])
        out = swiglu_expert(x[rows], w1, w3, w2)
        for r, (t, j) in enumerate(sel):
            y[pos[t]] += weights[t, j] * out[r]
    return y


def combine_per_token(x, weights, idx, disp, load_expert, tokens,
                      shared_out=None):
    """Per-token form: for each token, for each of its k choices, add
    p~ * Expert(x) unless that pair was dropped.  [SA] moe_forward step 4;
    [DD] section 4.3 (MoEWithSharedExpert: shared sum plus routed sum);
    [L17] section 2.4 (a dropped pair adds nothing)."""
    x = _f64(x)
    tok = np.asarray(tokens)
    y = np.zeros((len(tok), x.shape[1]))
    if shared_out is not None:
        y += _f64(shared_out)
    for i, t in enumerate(tok):
        for j in range(idx.shape[1]):
            if disp["drop"][t, j]:
                continue
            w1, w3, w2 = load_expert(int(idx[t, j]))
            y[i] += weights[t, j] * swiglu_expert(x[t:t + 1], w1, w3, w2)[0]
    return y


# --------------------------------------------------------------- statistics --

def load_balance_loss(f, P):
    """L_balance = E * sum_i f_i * P_i (alpha = 1).  [RM] section 3.2."""
    f = _f64(f)
    return float(f.shape[-1] * np.sum(f * _f64(P)))


def aux_stats(logits, counts, T, k, cap):
    """f_i, P_i, L_balance, z-loss and drop rate of one routed batch.

    f_i = (1/N) sum_t 1[t routed to i] with N = T, counted before the drop
    ([RM] section 3.2, so sum_i f_i = k); P_i = (1/N) sum_t p_{t,i};
    z = mean_t (logsumexp_i g_{t,i})^2 ([SA] router_z_loss, [DD] section 3.2,
    beta = 1); drop rate = dropped pairs / (T k) ([RM] section 4.3), where
    expert i drops max(0, counts_i - cap)."""
    g = _f64(logits)
    counts = np.asarray(counts, dtype=np.int64)
    f = counts / float(T)
    P = softmax(g).sum(axis=0) / float(T)
    lse = logsumexp(g)
    z = float(np.mean(lse * lse))
    dropped = int(np.maximum(counts - cap, 0).sum())
    return {"f": f, "P": P, "L_balance": load_balance_loss(f, P),
            "z_loss": z, "drop_rate": dropped / float(T * k)}


# ---------------------------------------------------------------- the layer --

def layer_forward(x, w_gate, k, CF, load_expert, E, E_shared=0,
                  load_shared=None, tokens=None, mode="grouped"):
    """Whole forward of one MoE layer, the order the pages give:
    route ([RM] 2.1) -> count and capacity-clip ([L17] 2.2, 2.4) ->
    experts and weighted sum plus always-on shared experts ([RM] 2.2,
    [L17] 5.2) -> statistics ([RM] 3.2, 4.3; [SA] router_z_loss).

    tokens: optional subset of token indices whose outputs are computed
    (routing, dispatch and statistics always cover all T tokens)."""
    x = _f64(x)
    T = x.shape[0]
    r = route(x, w_gate, k)
    counts = expert_counts(r["idx"], E)
    cap = capacity(T, E, k, CF)
    disp = dispatch(r["idx"], E, cap)
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    shared = None
    if E_shared:
        shared = np.zeros((len(tok), x.shape[1]))
        for s in range(E_shared):
            w1, w3, w2 = load_shared(s)
            shared += swiglu_expert(x[tok], w1, w3, w2)
    if mode == "grouped":
        y = combine_grouped(x, r["weights"], r["idx"], disp, load_expert, E,
                            tokens=tok, shared_out=shared)
    elif mode == "per_token":
        y = combine_per_token(x, r["weights"], r["idx"], disp, load_expert,
                              tok, shared_out=shared)
    else:
        raise ValueError(mode)
    stats = aux_stats(r["logits"], counts, T, k, cap)
    out = dict(r)
    out.update(counts=counts, cap=cap, y=y, tokens=tok, **disp)
    out.update(stats)
    return out


# ------------------------------------------------------------ backward (N2) --

def silu_grad(z):
    """d/dz SiLU(z) = sigma(z) (1 + z (1 - sigma(z)))."""
    z = _f64(z)
    sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def swiglu_expert_backward(xr, w1, w3, w2, dout):
    """Chain rule through Expert(x) = (SiLU(x W1) (*) x W3) W2 for rows xr
    and output gradient dout (storage layouts w1, w3 [F, d], w2 [d, F]).
    Returns dx, dw1, dw3, dw2 (same layouts)."""
    xr, w1, w3, w2, dout = (_f64(a) for a in (xr, w1, w3, w2, dout))
    a = xr @ w1.T
    b = xr @ w3.T
    s = silu(a)
    h = s * b
    dh = dout @ w2                     # [n, F]
    dw2 = dout.T @ h                   # [d, F]
    da = dh * b * silu_grad(a)
    db = dh * s
    dw1 = da.T @ xr                    # [F, d]
    dw3 = db.T @ xr
    dx = da @ w1 + db @ w3
    return dx, dw1, dw3, dw2


def layer_backward(x, w_gate, k, CF, load_expert, E, dy, alpha=0.0, beta=0.0,
                   E_shared=0, load_shared=None):
    """Gradients of L = sum(dy * y) + alpha * L_balance + beta * z_loss of
    one layer with respect to x, W_gate and every expert's weights.

    Routes (the pages'): y_t = sum_s Shared_s(x_t) + sum_{kept j} p~_tj
    o_tj; p~_t = softmax of the token's selected logits ([RM] 2.1), so
    dg_tS = p~ (dp~ - <p~, dp~>) over the selected set; a dropped pair has
    dp~ = 0 and no expert gradient ([L17] 2.4); L_balance = E sum f_i P_i
    with f_i constant and dL/dp_ti = alpha E f_i / T through softmax(g_t)
    ([RM] 3.4, [L17] 3.2); z = mean_t lse_t^2 gives dg_t = 2 beta lse_t
    p_t / T ([SA] router_z_loss); finally dW_gate = x^T dg and dx += dg
    W_gate^T."""
    x = _f64(x)
    dy = _f64(dy)
    wg = _f64(w_gate)
    T, d = x.shape
    r = route(x, wg, k)
    counts = expert_counts(r["idx"], E)
    cap = capacity(T, E, k, CF)
    disp = dispatch(r["idx"], E, cap)
    kept = disp["drop"] == 0
    pt = r["weights"]
    dx = np.zeros_like(x)
    dpt = np.zeros_like(pt)
    dws = []
    for e in range(E):
        tt, jj = np.nonzero((r["idx"] == e) & kept)
        w1, w3, w2 = (_f64(a) for a in load_expert(e))
        if len(tt) == 0:
            dws.append((np.zeros_like(w1), np.zeros_like(w3), np.zeros_like(w2)))
            continue
        out = swiglu_expert(x[tt], w1, w3, w2)
        dpt[tt, jj] = np.sum(dy[tt] * out, axis=1)
        dxe, dw1, dw3, dw2 = swiglu_expert_backward(x[tt], w1, w3, w2,
                                                    pt[tt, jj][:, None] * dy[tt])
        dx[tt] += dxe                  # a token picks an expert at most once
        dws.append((dw1, dw3, dw2))
    dshared = []
    for s_ in range(E_shared):
        dxs, dw1, dw3, dw2 = swiglu_expert_backward(x, *load_shared(s_), dy)
        dx += dxs
        dshared.append((dw1, dw3, dw2))
    dg = router_logit_grad(r, counts, dpt, E, alpha, beta)
    dx += dg @ wg.T
    return {"dx": dx, "dw_gate": x.T @ dg, "dw": dws, "dw_shared": dshared,
            "dtopk_w": dpt, "dg": dg, "route": r, "disp": disp, "counts": counts}


def router_logit_grad(r, counts, dpt, E, alpha, beta):
    """dL/dg for all tokens from the routing r, the per-expert counts and
    dp~ (dL/dp~ per (token, choice), 0 for a dropped pair): the selected
    softmax ([RM] 2.1), the balance loss through P_i ([RM] 3.4) and the
    z-loss ([SA] router_z_loss), as layer_backward states them."""
    pt = r["weights"]
    p = r["probs"]
    T = p.shape[0]
    dg = np.zeros((T, E))
    inner = np.sum(pt * dpt, axis=1, keepdims=True)
    np.add.at(dg, (np.arange(T)[:, None], r["idx"]), pt * (dpt - inner))
    c = alpha * E * (counts / float(T)) / float(T)
    dg += p * (c[None, :] - (p * c[None, :]).sum(axis=1, keepdims=True))
    dg += beta * 2.0 * r["lse"][:, None] * p / float(T)
    return dg


def layer_backward_sampled(x, w_gate, k, CF, load_expert, E, dy, alpha, beta, tokens, units,
                           E_shared=0, load_shared=None, shared_units=()):
    """The gradients of layer_backward at a sample, for layers too large to
    hold every weight gradient on the host: dx at the given tokens; for each
    (e, f) in units, row f of dW1 and dW3 and column f of dW2 of routed
    expert e (shared_units: the same for shared experts); dW_gate and dp~ in
    full (dp~ needs every expert output).

    Hidden unit f of a SwiGLU expert depends only on W1[f], W3[f] and
    W2[:, f], so the gradients of those weights are those of the expert cut
    down to the single unit f, which swiglu_expert_backward gives."""
    x = _f64(x)
    dy = _f64(dy)
    wg = _f64(w_gate)
    tokens = np.asarray(tokens)
    T, d = x.shape
    r = route(x, wg, k)
    counts = expert_counts(r["idx"], E)
    disp = dispatch(r["idx"], E, capacity(T, E, k, CF))
    kept = disp["drop"] == 0
    pt = r["weights"]
    dx = np.zeros((len(tokens), d))
    dpt = np.zeros_like(pt)
    where = {int(t): i for i, t in enumerate(tokens)}
    dw_units = {}
    for e in range(E):
        tt, jj = np.nonzero((r["idx"] == e) & kept)
        mine = [(e_, f) for (e_, f) in units if e_ == e]
        if len(tt) == 0:
            for (_, f) in mine:
                dw_units[(e, f)] = (np.zeros(d), np.zeros(d), np.zeros(d))
            continue
        w1, w3, w2 = (_f64(a) for a in load_expert(e))
        dpt[tt, jj] = np.sum(dy[tt] * swiglu_expert(x[tt], w1, w3, w2), axis=1)
        dout = pt[tt, jj][:, None] * dy[tt]
        sel = np.array([i for i, t in enumerate(tt) if int(t) in where], dtype=np.int64)
        if len(sel):
            dxe = swiglu_expert_backward(x[tt[sel]], w1, w3, w2, dout[sel])[0]
            for i, row in zip(sel, dxe):
                dx[where[int(tt[i])]] += row
        for (_, f) in mine:
            _, g1, g3, g2 = swiglu_expert_backward(x[tt], w1[f:f + 1], w3[f:f + 1],
                                                   w2[:, f:f + 1], dout)
            dw_units[(e, f)] = (g1[0], g3[0], g2[:, 0])
    dws_units = {}
    for s_ in range(E_shared):
        w1, w3, w2 = (_f64(a) for a in load_shared(s_))
        dx += swiglu_expert_backward(x[tokens], w1, w3, w2, dy[tokens])[0]
        for (s2, f) in shared_units:
            if s2 == s_:
                _, g1, g3, g2 = swiglu_expert_backward(x, w1[f:f + 1], w3[f:f + 1],
                                                       w2[:, f:f + 1], dy)
                dws_units[(s_, f)] = (g1[0], g3[0], g2[:, 0])
    dg = router_logit_grad(r, counts, dpt, E, alpha, beta)
    dx += dg[tokens] @ wg.T
    return {"dx": dx, "dw_units": dw_units, "dws_units": dws_units, "dw_gate": x.T @ dg,
            "dtopk_w": dpt, "dg": dg, "route": r, "disp": disp, "counts": counts}
