"""GPU parity of the backward pass (moe_combine_backward,
moe_expert_ffn_backward, moe_route_backward) against the oracle's
layer_backward on the same bits: every gradient within the bf16 bounds
(max error <= 2e-2 max|ref|, sum|err| / sum|ref| <= 5e-3)."""
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


def _close(name, got, ref):
    mx, mr = H.y_errors(np.asarray(got, dtype=np.float64), ref)
    H.log(f"  {name}: max_err={mx:.2e} mean_rel={mr:.2e}")
    assert mx <= 2e-2, f"{name}: max error {mx:.3e} > 2e-2 of max|ref|"
    assert mr <= 5e-3, f"{name}: mean relative error {mr:.3e} > 5e-3"


def _backward_case(cfg, alpha, beta, seed=9):
    import top_routing_expert_softmax_amd as M
    H.log(f"backward: {cfg}")
    inp = H.LayerInputs(cfg)
    dd = inp.dev
    b = H.run_gpu(inp)
    rng = np.random.default_rng(seed)
    dy32 = rng.standard_normal((cfg.T, cfg.d_model)).astype(np.float32)
    dy_dev = torch.from_numpy(dy32).cuda().to(torch.bfloat16)
    dy = dy_dev.float().cpu().numpy().astype(np.float64)
    dx, dwg, dw, dws = M.layer_backward(inp.x_dev, inp.wg_dev, dd["w1"], dd["w3"], dd["w2"],
                                        cfg.k, dy_dev, alpha, beta, b, dd.get("ws1"),
                                        dd.get("ws3"), dd.get("ws2"))
    torch.cuda.synchronize()
    g = O.layer_backward(inp.x, inp.wg, cfg.k, cfg.CF, inp.load_routed, cfg.E, dy, alpha, beta,
                         cfg.E_shared, inp.load_shared if cfg.E_shared else None)
    assert np.array_equal(b.topk_idx.cpu().numpy(), g["route"]["idx"])
    _close("dx", dx.float().cpu().numpy(), g["dx"])
    _close("dw_gate", dwg.cpu().numpy(), g["dw_gate"])
    for m, name in enumerate(("dw1", "dw3", "dw2")):
        got = dw[m].cpu().numpy()
        ref = np.stack([g["dw"][e][m] for e in range(cfg.E)])
        _close(name, got, ref)
        if cfg.E_shared:
            _close("shared " + name, dws[m].cpu().numpy(),
                   np.stack([g["dw_shared"][s][m] for s in range(cfg.E_shared)]))


def test_backward_small_with_drops_and_shared():
    cfg = get_config("dsmoe16b_prefill", T=300, d_model=256, E=8, E_shared=1, k=2, d_ff=320,
                     CF=1.0)
    _backward_case(cfg, alpha=0.1, beta=0.01)


def test_backward_mid_size():
    cfg = get_config("mixtral_prefill", T=1024, d_model=1024, E=8, k=2, d_ff=2048, CF=1.25)
    _backward_case(cfg, alpha=0.01, beta=0.001)
