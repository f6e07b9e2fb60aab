"""GPU parity of moe_route on its own, across both router kernels: the
matrix-core one (bf16, E a multiple of 8; with few tokens d is split over
blocks and a select kernel adds the splits) and the fp32 FMA one (fp32,
other E).  Logits
and chosen experts bit-exact against the oracle, weights within 2e-6.

The cases reach every expert padding of the matrix-core kernel (E rounded
up to 16, 32, 64, 128, 256), both token tilings, a last token tile that is
partly past T, d ranges that do not divide evenly over the block's waves
(a wave with a short last batch, a wave with no k-steps), and E not a power
of two (staged columns past E)."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import get_config, router_inputs, storage_bits

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_routing_expert_softmax_amd as M
    M.lib()


ROUTER_CASES = {
    # E = 8 (padded to 16), 1101 tokens: 69 blocks of 16, the last holding
    # 13 (its last group of four tokens holds one); d = 1088 is 34 k-steps
    # over 8 waves (five each, the seventh four, the last none)
    "mfma_E8_ragged": ("mixtral_prefill", dict(T=1101, d_model=1088, E=8, k=2)),
    # E = 24 (padded to 32), 8200 tokens in blocks of 32 (the last holds 8)
    "mfma_E24_tiles32": ("mixtral_prefill", dict(T=8200, d_model=512, E=24, k=3)),
    # E = 40 (padded to 64: three of eight staged chunks per row unused);
    # the last block holds 14 tokens
    "mfma_E40": ("dsmoe16b_prefill", dict(T=1502, d_model=640, E=40, E_shared=0, k=4)),
    # E = 128, eight per token
    "mfma_E128": ("dsv3_decode", dict(T=2048, d_model=2048, E=128, k=8)),
    # E = 160 (padded to 256): three waves per block over 32 k-steps
    "mfma_E160": ("dsv3_decode", dict(T=1031, d_model=1024, E=160, k=6)),
    # E = 256 in blocks of 32 tokens: two waves per block
    "mfma_E256_tiles32": ("dsv3_decode", dict(T=8208, d_model=768, E=256, k=8)),
    # few tokens: the matrix-core kernel with d split over blocks, then the
    # select kernel; 37 tokens (the last tile holds 5), 50 k-steps in 10
    # splits of 5, one k-step per wave
    "mfma_split_E24": ("mixtral_prefill", dict(T=37, d_model=1600, E=24, k=3)),
    # split path with 256 experts and 20 tokens
    "mfma_split_E256": ("dsv3_decode", dict(T=20, d_model=1024, E=256, k=8)),
    # E not a multiple of 8 in bf16: the fp32 FMA kernel
    "fma_bf16_E12": ("mixtral_prefill", dict(T=1100, d_model=512, E=12, k=2)),
    # fp32 activations and weights: the fp32 FMA kernel
    "fma_f32_E64": ("tiny_f32", dict(T=1100, d_model=256, E=64, k=4)),
}


@pytest.mark.parametrize("label", list(ROUTER_CASES))
def test_route_matches_oracle(label):
    import top_routing_expert_softmax_amd as M
    base, over = ROUTER_CASES[label]
    cfg = get_config(base, **over)
    T, d, E, k = cfg.T, cfg.d_model, cfg.E, cfg.k
    H.log(f"route {label}: dtype={cfg.dtype} T={T} d={d} E={E} k={k}")
    x, wg = router_inputs(cfg)
    x_dev = H.to_device(cfg, storage_bits(cfg, x))
    wg_dev = H.to_device(cfg, storage_bits(cfg, wg))
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    # the split path needs the workspace; the large-T path takes none
    nbytes = M.moe_workspace_size(T, d, E, 0, k, 64, x_dev.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if T < 1024 else None
    M.moe_route(x_dev, wg_dev, k, logits, idx, w, ws)
    torch.cuda.synchronize()
    r = O.route(x, wg, k)
    assert np.array_equal(logits.cpu().numpy().astype(np.float64), r["logits"]), "logits differ"
    assert np.array_equal(idx.cpu().numpy(), r["idx"]), "chosen experts differ"
    assert np.max(np.abs(w.cpu().numpy() - r["weights"])) <= 2e-6, "weights differ"


@pytest.mark.parametrize("E", [64, 128])
def test_route_all_ties_take_the_lowest_experts(E):
    """W_gate = 0 on the matrix-core path: every logit is 0, so each token
    takes experts 0..k-1 with weight 1/k (four tokens per wavefront for
    E = 64, one for E = 128)."""
    import top_routing_expert_softmax_amd as M
    T, d, k = 1030, 256, 6
    cfg = get_config("mixtral_prefill", T=T, d_model=d, E=E, k=k)
    x, _ = router_inputs(cfg)
    x_dev = H.to_device(cfg, storage_bits(cfg, x))
    wg_dev = torch.zeros((d, E), dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    M.moe_route(x_dev, wg_dev, k, logits, idx, w, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(logits).item() == 0
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(k), (T, 1)))
    np.testing.assert_allclose(w.cpu().numpy(), 1.0 / k, rtol=1e-6)


@pytest.mark.parametrize("T", [2048, 40])
def test_route_off_the_grid_within_the_fp32_sum_bound(T):
    """Seeded Gaussian bf16 x and W_gate (not on the dyadic grid), both
    matrix-core paths (T = 2048 in one pass, T = 40 with d split over
    blocks).  Every logit is within the bound of a d-term fp32 sum,
    gamma_d * sum_i |x_ti w_ie| with gamma_d = d u / (1 - d u), u = 2^-24,
    of the oracle's fp64 value; where the k-th and (k+1)-th largest oracle
    logits of a token are further apart than twice that bound, the chosen
    experts are the oracle's."""
    import top_routing_expert_softmax_amd as M
    d, E, k = 1024, 64, 6
    rng = np.random.default_rng(1234 + T)
    bf = torch.bfloat16
    x_t = torch.from_numpy(rng.standard_normal((T, d), dtype=np.float32)).to(bf)
    w_t = torch.from_numpy((rng.standard_normal((d, E), dtype=np.float32) * 0.05)).to(bf)
    x = x_t.float().numpy().astype(np.float64)
    wg = w_t.float().numpy().astype(np.float64)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(M.moe_workspace_size(T, d, E, 0, k, 64, bf), dtype=torch.uint8, device="cuda")
    M.moe_route(x_t.cuda(), w_t.cuda(), k, logits, idx, w, ws)
    torch.cuda.synchronize()
    ref = O.router_logits(x, wg)
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    bound = gamma * (np.abs(x) @ np.abs(wg))
    err = np.abs(logits.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= bound), float(np.max(err / bound))
    srt = np.sort(ref, axis=1)[:, ::-1]
    clear = (srt[:, k - 1] - srt[:, k]) > 2 * bound.max(axis=1)
    assert clear.mean() > 0.5                  # most tokens are decided
    got = np.sort(idx.cpu().numpy(), axis=1)
    want = np.sort(O.route(x, wg, k)["idx"], axis=1)
    assert np.array_equal(got[clear], want[clear]), "chosen experts differ on a clear token"
