"""GPU parity of the FP8 expert weights (moe_quantize_fp8,
moe_expert_ffn_fp8): the codes and row scales bit-exact against the
oracle's independent quantiser, and the decode layer's y against the oracle
computing with the dequantised weights, to the bf16 bounds."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import bf16_bits_to_f32, get_config

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_routing_expert_softmax_amd as M
    M.lib()


def _quantize_dev(w_dev):
    import top_routing_expert_softmax_amd as M
    cols = w_dev.shape[-1]
    codes = torch.empty(w_dev.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty(w_dev.shape[:-1], dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(w_dev.reshape(-1, cols), codes, scales)
    return codes, scales


def test_quantizer_matches_oracle():
    rng = np.random.default_rng(0)
    for rows, cols in ((64, 1024), (3, 7168), (257, 64)):
        w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
        w[rng.integers(0, rows)] = 0.0                       # a zero row
        w[0, :5] = [1e-30, -3e-7, 0.5, -0.5, 2.0]            # subnormal codes and a big outlier
        bits = np.asarray(torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy())
        wb = bf16_bits_to_f32(bits.view(np.uint16))
        for dev in (torch.from_numpy(bits).cuda().view(torch.bfloat16),
                    torch.from_numpy(wb).cuda()):
            codes, scales = _quantize_dev(dev)
            torch.cuda.synchronize()
            want_c, want_s = O.quantize_fp8_rows(wb)
            assert np.array_equal(scales.cpu().numpy(), want_s), (rows, cols, dev.dtype)
            assert np.array_equal(codes.cpu().numpy(), want_c), (rows, cols, dev.dtype)


def _fp8_layer(cfg, tokens=None, code_experts=None):
    import top_routing_expert_softmax_amd as M
    H.log(f"fp8 layer: {cfg}")
    inp = H.LayerInputs(cfg)
    T, d, E, Es, k, F = cfg.T, cfg.d_model, cfg.E, cfg.E_shared, cfg.k, cfg.d_ff
    dd = inp.dev
    q = {kind: _quantize_dev(dd[kind]) for kind in dd}
    b = M.MoELayerBuffers(T, d, E, Es, k, F, torch.bfloat16)
    M.moe_route(inp.x_dev, inp.wg_dev, k, b.logits, b.topk_idx, b.topk_w, b.ws)
    M.moe_permute(b.topk_idx, inp.x_dev, E, cfg.CF, b.counts, b.offsets, b.token_of_row,
                  b.row_of_pair, b.drop_mask, b.x_perm, b.ws)
    sh = {}
    if Es:
        sh = dict(sq1=q["ws1"][0], sq3=q["ws3"][0], sq2=q["ws2"][0], ss1=q["ws1"][1],
                  ss3=q["ws3"][1], ss2=q["ws2"][1], y_shared=b.y_shared)
    M.moe_expert_ffn_fp8(T, k, b.x_perm, b.offsets, inp.x_dev, q["w1"][0], q["w3"][0],
                         q["w2"][0], q["w1"][1], q["w3"][1], q["w2"][1], b.y_perm, b.ws, **sh)
    M.moe_combine(b.y_perm, b.y_shared, b.row_of_pair, b.topk_w, b.y)
    torch.cuda.synchronize()
    r, counts, cap, disp, stats = H.oracle_routing(inp)
    assert np.array_equal(b.topk_idx.cpu().numpy(), r["idx"])
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    need = set(int(e) for e in np.unique(r["idx"][toks]))
    check = need if code_experts is None else need | set(code_experts)
    deq = {}

    def oracle_expert(kind_prefix, e):
        out = []
        for kind in ("1", "3", "2"):
            name = kind_prefix + kind
            wv = inp.host_expert(name, e)
            c, s = O.quantize_fp8_rows(wv)
            if code_experts is None or e in check:
                gc, gs = q[name][0][e].cpu().numpy(), q[name][1][e].cpu().numpy()
                assert np.array_equal(gs, s) and np.array_equal(gc, c), (name, e)
            out.append(O.dequantize_fp8_rows(c, s))
        return tuple(out)

    for e in sorted(need):
        deq[e] = oracle_expert("w", e)
    ref = np.zeros((len(toks), d))
    for s_ in range(Es):
        ref += O.swiglu_expert(inp.x[toks], *oracle_expert("ws", s_))
    for i, t in enumerate(toks):
        for j in range(k):
            if disp["drop"][t, j]:
                continue
            e = int(r["idx"][t, j])
            ref[i] += r["weights"][t, j] * O.swiglu_expert(inp.x[t:t + 1], *deq[e])[0]
    mx, mr = H.check_y(cfg, b.y.float().cpu().numpy()[toks], ref)
    H.log(f"fp8 layer {cfg.name}: experts checked={len(need)} max_err={mx:.2e} mean_rel={mr:.2e}")


def test_fp8_decode_layer_small():
    cfg = get_config("dsv3_decode", T=40, d_model=1024, E=32, E_shared=1, k=4, d_ff=512)
    _fp8_layer(cfg)


def test_fp8_decode_layer_full_size():
    """DeepSeek-V3 decode shape (every touched expert streamed once as FP8);
    y on two tokens, codes checked on their experts and the shared one."""
    cfg = get_config("dsv3_decode")
    _fp8_layer(cfg, tokens=[0, 37])


@pytest.mark.parametrize("counts,T,k", [
    # 1 .. 4 rows read the token rows from LDS (FP8 limit 4), 5 from L2,
    # 16 and 17 rows one and two token groups, 64 the largest streamed
    ([0, 1, 2, 3, 4, 5, 16, 17, 64, 0, 7], 64, 4),
    # T = 4: the shared expert's all-token segment is staged too
    ([0, 1, 4, 2, 3], 4, 3),
])
def test_fp8_stream_segments_at_the_staging_limits(counts, T, k):
    """moe_expert_ffn_fp8 on chosen decode-sized segments around the LDS
    staging of token rows, d = 320 and F = 192 (rows of 640 and 384 bytes;
    K loops of 5 and 3 steps of 64: whole batches and a remainder), against
    the oracle computing with the dequantised weights."""
    import top_routing_expert_softmax_amd as M
    d_model, d_ff = 320, 192
    cfg = get_config("dsv3_decode", T=T, d_model=d_model, E=len(counts), E_shared=1, k=k,
                     d_ff=d_ff, CF=None)
    H.log(f"fp8 staging limits: counts={counts} T={T} k={k}")
    inp = H.LayerInputs(cfg)
    dd = inp.dev
    q = {kind: _quantize_dev(dd[kind]) for kind in dd}
    R = sum(counts)
    src = np.arange(R) % T
    xp = torch.zeros((T * k, d_model), dtype=torch.bfloat16, device="cuda")
    xp[:R] = inp.x_dev[torch.from_numpy(src).cuda()]
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32,
                        device="cuda")
    E = len(counts)
    ws = torch.empty(M.moe_workspace_size(T, d_model, E, 1, k, d_ff, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    yp = torch.empty((T * k, d_model), dtype=torch.bfloat16, device="cuda")
    ysh = torch.empty((1, T, d_model), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_fp8(T, k, xp, offs, inp.x_dev, q["w1"][0], q["w3"][0], q["w2"][0],
                         q["w1"][1], q["w3"][1], q["w2"][1], yp, ws, sq1=q["ws1"][0],
                         sq3=q["ws3"][0], sq2=q["ws2"][0], ss1=q["ws1"][1], ss3=q["ws3"][1],
                         ss2=q["ws2"][1], y_shared=ysh)
    torch.cuda.synchronize()

    def deq(name, e):
        c, s = O.quantize_fp8_rows(inp.host_expert(name, e))
        return O.dequantize_fp8_rows(c, s)

    x64 = inp.x.astype(np.float64)
    o = np.concatenate([[0], np.cumsum(counts)])
    got, ref = [], []
    for e in range(E):
        if counts[e] == 0:
            continue
        got.append(yp[o[e]:o[e + 1]].float().cpu().numpy())
        ref.append(O.swiglu_expert(x64[src[o[e]:o[e + 1]]], deq("w1", e), deq("w3", e),
                                   deq("w2", e)))
    got.append(ysh[0].float().cpu().numpy())
    ref.append(O.swiglu_expert(x64, deq("ws1", 0), deq("ws3", 0), deq("ws2", 0)))
    mx, mr = H.check_y(cfg, np.concatenate(got), np.concatenate(ref))
    H.log(f"  y: max_err={mx:.2e} mean_rel={mr:.2e}")
