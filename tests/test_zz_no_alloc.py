"""moe_expert_ffn_noalloc (the library's fixed device scratch, no workspace)
against moe_expert_ffn on the same inputs, through the C ABI: two calls in a
row on decode-shaped layers, the second smaller than the first, so the
scratch holds the first call's contents when the second one starts.  The
two entry points run the same kernels on the same layout, so their outputs
must be identical bit for bit."""
import numpy as np
import pytest
import torch

from workloads import get_config

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402

# (base config, overrides): each pair runs larger first, then smaller
PAIRS = {
    # weight-streamed segments only (T <= 64), one shared expert
    "streamed": (("dsv3_decode", dict(T=64, d_model=1024, E=64, E_shared=1, k=6, d_ff=512)),
                 ("dsv3_decode", dict(T=16, d_model=512, E=32, E_shared=1, k=4, d_ff=256))),
    # T > 64 with T*k < 64*E: streamed segments beside 128-row tiles (tile
    # table in the scratch), then a smaller streamed-only call
    "mixed_tiles": (("skewed_train", dict(T=200, d_model=256, E=16, E_shared=1, k=2, d_ff=256,
                                          CF=None, zipf_tau=1.0)),
                    ("dsv3_decode", dict(T=8, d_model=256, E=16, E_shared=0, k=2, d_ff=128))),
    # the fp32 tiles
    "f32": (("tiny_f32", dict(T=200, d_model=192, E=5, k=2, d_ff=320, CF=1.0, E_shared=1)),
            ("tiny_f32", {})),
}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_routing_expert_softmax_amd as M
    M.lib()


def _layer(base, over):
    cfg = get_config(base, **over)
    inp = H.LayerInputs(cfg, keep_host=False)
    return cfg, inp, H.run_gpu(inp)


@pytest.mark.parametrize("pair", list(PAIRS))
def test_noalloc_ffn_equals_the_workspace_entry_point(pair):
    import top_routing_expert_softmax_amd as M
    runs = [_layer(*spec) for spec in PAIRS[pair]]
    for i, (cfg, inp, b) in enumerate(runs):
        H.log(f"noalloc {pair} call {i}: {cfg}")
        d = inp.dev
        R = int(b.offsets[-1].item())
        yp = torch.full_like(b.y_perm, float("nan"))
        ysh = torch.full_like(b.y_shared, float("nan")) if cfg.E_shared else None
        M.moe_expert_ffn_noalloc(cfg.T, cfg.k, b.x_perm, b.offsets, inp.x_dev, d["w1"], d["w3"],
                                 d["w2"], d.get("ws1"), d.get("ws3"), d.get("ws2"), yp, ysh)
        torch.cuda.synchronize()
        assert torch.equal(yp[:R], b.y_perm[:R]), f"{pair} call {i}: y_perm differs"
        if cfg.E_shared:
            assert torch.equal(ysh, b.y_shared), f"{pair} call {i}: y_shared differs"
        assert R > 0 and not torch.isnan(yp[:R].float()).any()
