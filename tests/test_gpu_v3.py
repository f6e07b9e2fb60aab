"""GPU parity of the DeepSeek-V3 gate (moe_route_v3, moe_update_bias)
against the oracle: logits bit-exact, chosen experts bit-exact (both sides
decide in fp32 on the same fp32 affinities), weights within 2e-6 of the
route scale; the bias step bit-exact; and a whole layer routed by the gate."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import get_config, router_inputs, storage_bits

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "v3_gate_hand.json")))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_routing_expert_softmax_amd as M
    M.lib()


def _run_v3(cfg, bias, n_groups, topk_groups, scale, zero_gate=False):
    import top_routing_expert_softmax_amd as M
    x, wg = router_inputs(cfg)
    if zero_gate:
        wg = np.zeros_like(wg)
    T, E, k = cfg.T, cfg.E, cfg.k
    x_dev = H.to_device(cfg, storage_bits(cfg, x))
    wg_dev = H.to_device(cfg, storage_bits(cfg, wg))
    b_dev = torch.tensor(np.asarray(bias, dtype=np.float32), device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    nbytes = M.moe_workspace_size(T, cfg.d_model, E, 0, k, 64, x_dev.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    M.moe_route_v3(x_dev, wg_dev, b_dev, k, n_groups, topk_groups, scale, logits, idx, w, ws)
    torch.cuda.synchronize()
    r = O.v3_gate(O.router_logits(x, wg), bias, k, n_groups, topk_groups, scale)
    return logits.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), r


def _check(cfg, bias, n_groups, topk_groups, scale, label):
    H.log(f"v3 gate {label}: T={cfg.T} d={cfg.d_model} E={cfg.E} k={cfg.k} "
          f"groups={n_groups}/{topk_groups}")
    lg, idx, w, r = _run_v3(cfg, bias, n_groups, topk_groups, scale)
    assert np.array_equal(lg.astype(np.float64), r["logits"]), "logits differ"
    assert np.array_equal(idx, r["idx"]), "chosen experts differ"
    assert np.max(np.abs(w - r["weights"])) <= 2e-6 * scale, "weights differ"
    np.testing.assert_allclose(w.sum(axis=1), scale, rtol=1e-5)


V3_CASES = {
    # DeepSeek-V3 decode: 64 tokens, d split across blocks (two-kernel path)
    "dsv3_decode": ("dsv3_decode", {}, 8, 4, 2.5),
    # many tokens: one pass per 8 tokens; 8 groups of 8, keep 3
    "prefill_groups": ("dsmoe16b_prefill", dict(T=2048, d_model=1024, E=64, E_shared=0, k=6),
                       8, 3, 1.0),
    # small E, every group kept
    "all_groups": ("mixtral_prefill", dict(T=300, d_model=256, E=16, k=4), 4, 4, 1.5),
    # the DeepSeek-V3 gate at a prefill size: the matrix-core router with
    # 256 experts (three waves per block) and the gate in its epilogue
    "prefill_E256": ("dsv3_decode", dict(T=1100, d_model=1024), 8, 4, 2.5),
}


@pytest.mark.parametrize("label", list(V3_CASES))
def test_v3_gate_matches_oracle(label):
    base, over, ng, tg, scale = V3_CASES[label]
    cfg = get_config(base, **over)
    rng = np.random.default_rng(11)
    bias = rng.uniform(-0.1, 0.1, cfg.E).astype(np.float32)
    _check(cfg, bias, ng, tg, scale, label)


def test_v3_without_groups_or_bias_picks_the_softmax_experts():
    """One group, zero bias: the same ids as moe_route (sigmoid and softmax
    are both increasing in the logit)."""
    import top_routing_expert_softmax_amd as M
    cfg = get_config("mixtral_prefill", T=500, d_model=512, E=8, k=2)
    lg, idx, w, r = _run_v3(cfg, np.zeros(8, np.float32), 1, 1, 1.0)
    x, wg = router_inputs(cfg)
    x_dev = H.to_device(cfg, storage_bits(cfg, x))
    wg_dev = H.to_device(cfg, storage_bits(cfg, wg))
    logits = torch.empty((cfg.T, 8), dtype=torch.float32, device="cuda")
    idx2 = torch.empty((cfg.T, 2), dtype=torch.int32, device="cuda")
    w2 = torch.empty((cfg.T, 2), dtype=torch.float32, device="cuda")
    M.moe_route(x_dev, wg_dev, 2, logits, idx2, w2, None)
    torch.cuda.synchronize()
    assert np.array_equal(idx, idx2.cpu().numpy())
    assert np.array_equal(idx, r["idx"])


def test_v3_hand_example_on_device():
    """The hand-worked example (all logits 0, given biases) on every token."""
    c = GOLD["groups_by_top2"]
    cfg = get_config("mixtral_prefill", T=40, d_model=128, E=c["E"], k=c["k"])
    lg, idx, w, r = _run_v3(cfg, np.asarray(c["bias"], np.float32), c["n_groups"],
                            c["topk_groups"], c["route_scale"], zero_gate=True)
    assert np.all(lg == 0.0)
    assert np.all(idx == np.asarray(c["idx"])[None, :])
    np.testing.assert_allclose(w, np.broadcast_to(c["weights"], w.shape), rtol=1e-6)


def test_bias_step_matches_oracle():
    import top_routing_expert_softmax_amd as M
    rng = np.random.default_rng(4)
    for T, E, k in ((64, 256, 8), (1000, 64, 6), (4, 4, 2)):
        counts = rng.multinomial(T * k, np.full(E, 1.0 / E)).astype(np.int32)
        if E == 4:
            counts = np.array(GOLD["bias_step"]["counts"], dtype=np.int32)
        bias = rng.uniform(-0.2, 0.2, E).astype(np.float32)
        c_dev = torch.tensor(counts, device="cuda")
        b_dev = torch.tensor(bias, device="cuda")
        M.moe_update_bias(T, k, 1e-3, c_dev, b_dev)
        torch.cuda.synchronize()
        want = O.update_bias(counts, bias, T, k, 1e-3)
        assert np.array_equal(b_dev.cpu().numpy(), want), (T, E, k)


def test_layer_routed_by_the_v3_gate():
    """moe_route_v3 -> moe_permute -> moe_expert_ffn -> moe_combine against
    the oracle's dispatch and combine fed with the gate's choice (weights
    sum to 2.5, one shared expert, capacity drops on)."""
    import top_routing_expert_softmax_amd as M
    cfg = get_config("dsmoe16b_prefill", T=384, d_model=256, E=16, E_shared=1, k=4,
                     d_ff=256, CF=1.0)
    H.log(f"v3 layer: {cfg}")
    inp = H.LayerInputs(cfg)
    rng = np.random.default_rng(2)
    bias = rng.uniform(-0.05, 0.05, cfg.E).astype(np.float32)
    b = M.MoELayerBuffers(cfg.T, cfg.d_model, cfg.E, cfg.E_shared, cfg.k, cfg.d_ff,
                          torch.bfloat16)
    d = inp.dev
    M.moe_route_v3(inp.x_dev, inp.wg_dev, torch.tensor(bias, device="cuda"), cfg.k, 4, 2, 2.5,
                   b.logits, b.topk_idx, b.topk_w, b.ws)
    M.moe_permute(b.topk_idx, inp.x_dev, cfg.E, cfg.CF, b.counts, b.offsets, b.token_of_row,
                  b.row_of_pair, b.drop_mask, b.x_perm, b.ws)
    M.moe_expert_ffn(cfg.T, cfg.k, b.x_perm, b.offsets, inp.x_dev, d["w1"], d["w3"], d["w2"],
                     d["ws1"], d["ws3"], d["ws2"], b.y_perm, b.y_shared, b.ws)
    M.moe_combine(b.y_perm, b.y_shared, b.row_of_pair, b.topk_w, b.y)
    torch.cuda.synchronize()
    r = O.v3_gate(O.router_logits(inp.x, inp.wg), bias, cfg.k, 4, 2, 2.5)
    assert np.array_equal(b.topk_idx.cpu().numpy(), r["idx"])
    cap = O.capacity(cfg.T, cfg.E, cfg.k, cfg.CF)
    disp = O.dispatch(r["idx"], cfg.E, cap)
    assert np.array_equal(b.drop_mask.cpu().numpy(), disp["drop"])
    shared = O.swiglu_expert(inp.x, *inp.load_shared(0))
    ref = O.combine_grouped(inp.x, r["weights"], r["idx"], disp, inp.load_routed, cfg.E,
                            shared_out=shared)
    mx, mr = H.check_y(cfg, b.y.float().cpu().numpy(), ref)
    H.log(f"v3 layer: drops={int(disp['drop'].sum())} max_err={mx:.2e} mean_rel={mr:.2e}")
