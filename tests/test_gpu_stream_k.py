"""GPU parity of the weight-streaming kernels over K lengths.

The streaming kernels split a weight row's K steps into batches that the
four waves of a block take round robin, from a rotation of the batch order
that depends on the block, with the steps past the whole batches done by
one wave.  These cases choose d and F so that the number of whole batches
runs from none to several, with and without a remainder, for both weight
types (bf16: batches of four 32-wide steps; FP8: four 64-wide steps in
phase 1, two in phase 2), on segments of every token-group form (token
rows staged in LDS, one, two and three groups of 16 rows, and a shared
expert of all T tokens).  Every row of every segment is compared with the
oracle's SwiGLU expert ("CMU 11-868 Lecture 17" section 5.2), computed with
the dequantised weights for FP8."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import get_config

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402

COUNTS = [1, 3, 5, 16, 20, 40]
T, K_ROUTE, E_SHARED = 48, 2, 1


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_routing_expert_softmax_amd as M
    M.lib()


def _quantize(w_dev):
    import top_routing_expert_softmax_amd as M
    codes = torch.empty(w_dev.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty(w_dev.shape[:-1], dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(w_dev.reshape(-1, w_dev.shape[-1]), codes, scales)
    return codes, scales


# (d, F): whole batches of the bf16 kernel (d/32 or F/32 steps in batches
# of 4) and of the FP8 kernel (d/64 steps in batches of 4, F/64 in batches
# of 2) range over 0 .. 16, with remainders of 0 .. 3 steps
@pytest.mark.parametrize("weights", ["bf16", "fp8"])
@pytest.mark.parametrize("d_model,d_ff", [(64, 320), (192, 576), (576, 64), (1088, 1152)])
def test_stream_batches_over_k(weights, d_model, d_ff):
    import top_routing_expert_softmax_amd as M
    cfg = get_config("dsv3_decode", T=T, d_model=d_model, E=len(COUNTS), E_shared=E_SHARED,
                     k=K_ROUTE, d_ff=d_ff, CF=None)
    H.log(f"stream K batches: {weights} d={d_model} F={d_ff} counts={COUNTS}")
    inp = H.LayerInputs(cfg)
    E = len(COUNTS)
    R = sum(COUNTS)
    src = np.arange(R) % T
    xp = torch.zeros((T * K_ROUTE, d_model), dtype=torch.bfloat16, device="cuda")
    xp[:R] = inp.x_dev[torch.from_numpy(src).cuda()]
    o = np.concatenate([[0], np.cumsum(COUNTS)])
    offs = torch.tensor(o, dtype=torch.int32, device="cuda")
    ws = torch.empty(M.moe_workspace_size(T, d_model, E, E_SHARED, K_ROUTE, d_ff, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    yp = torch.empty((T * K_ROUTE, d_model), dtype=torch.bfloat16, device="cuda")
    ysh = torch.empty((E_SHARED, T, d_model), dtype=torch.bfloat16, device="cuda")
    dd = inp.dev
    if weights == "bf16":
        M.moe_expert_ffn(T, K_ROUTE, xp, offs, inp.x_dev, dd["w1"], dd["w3"], dd["w2"],
                         dd["ws1"], dd["ws3"], dd["ws2"], yp, ysh, ws)

        def expert(kinds, e):
            return tuple(inp.host_expert(kk, e).astype(np.float64) for kk in kinds)
    else:
        q = {kind: _quantize(dd[kind]) for kind in ("w1", "w3", "w2", "ws1", "ws3", "ws2")}
        M.moe_expert_ffn_fp8(T, K_ROUTE, xp, offs, inp.x_dev, q["w1"][0], q["w3"][0],
                             q["w2"][0], q["w1"][1], q["w3"][1], q["w2"][1], yp, ws,
                             sq1=q["ws1"][0], sq3=q["ws3"][0], sq2=q["ws2"][0],
                             ss1=q["ws1"][1], ss3=q["ws3"][1], ss2=q["ws2"][1], y_shared=ysh)

        def expert(kinds, e):
            return tuple(O.dequantize_fp8_rows(*O.quantize_fp8_rows(inp.host_expert(kk, e)))
                         for kk in kinds)
    torch.cuda.synchronize()
    x64 = inp.x.astype(np.float64)
    got, ref = [], []
    for e in range(E):
        got.append(yp[o[e]:o[e + 1]].float().cpu().numpy())
        ref.append(O.swiglu_expert(x64[src[o[e]:o[e + 1]]], *expert(("w1", "w3", "w2"), e)))
    got.append(ysh[0].float().cpu().numpy())
    ref.append(O.swiglu_expert(x64, *expert(("ws1", "ws3", "ws2"), 0)))
    mx, mr = H.check_y(cfg, np.concatenate(got), np.concatenate(ref))
    H.log(f"  y: max_err={mx:.2e} mean_rel={mr:.2e}")
