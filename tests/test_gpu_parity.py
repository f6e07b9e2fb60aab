"""GPU parity: the HIP layer (through the C ABI) against the fp64 oracle.

Integer outputs (top-k ids, counts, offsets, permutation, drop mask) and the
logits must match bit for bit; weights within 2e-6; y within the bounds the
layer promises (fp32: max error <= 1e-4 max|ref|; bf16: max error <= 2e-2
max|ref| and sum|err|/sum|ref| <= 5e-3); statistics within 1e-5 relative.
"""
import numpy as np
import pytest
import torch

from workloads import get_config

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_routing_expert_softmax_amd as M
    M.lib()      # raises if the HIP library is missing: no silent fallback


def _full_check(cfg, label):
    H.log(f"case {label}: {cfg}")
    inp = H.LayerInputs(cfg)
    g = H.host(H.run_gpu(inp))
    r, counts, cap, disp, stats = H.oracle_routing(inp)
    H.check_routing(g, r, counts, disp)
    ref = H.oracle_y(inp, r, disp, np.arange(cfg.T))
    mx, mr = H.check_y(cfg, g["y"], ref)
    H.check_stats(g, stats)
    H.log(f"case {label}: R={g['R']} drop={stats['drop_rate']:.4f} max_err={mx:.2e} mean_rel={mr:.2e}")


SMALL_CASES = {
    # name: (base config, overrides)
    "tiny_f32": ("tiny_f32", {}),
    "f32_ragged": ("tiny_f32", dict(T=200, d_model=192, E=5, k=2, d_ff=320, CF=1.0, E_shared=1)),
    "bf16_ragged_shared": ("dsmoe16b_prefill", dict(T=300, d_model=192, E=6, E_shared=1, k=2,
                                                     d_ff=320, CF=1.0)),
    "bf16_multi_tile": ("mixtral_prefill", dict(T=700, d_model=256, E=4, k=2, d_ff=512,
                                                CF=1.25)),
    "bf16_two_shared_k6": ("dsmoe16b_prefill", dict(T=260, d_model=128, E=16, E_shared=2, k=6,
                                                    d_ff=192, CF=1.25)),
    "bf16_T1": ("dsv3_decode", dict(T=1, d_model=256, E=32, E_shared=1, k=8, d_ff=128)),
    "bf16_E1_k1": ("mixtral_prefill", dict(T=150, d_model=128, E=1, k=1, d_ff=128, CF=None)),
    "bf16_empty_experts": ("dsv3_decode", dict(T=5, d_model=128, E=64, E_shared=0, k=2,
                                               d_ff=128)),
    "bf16_skew_drop": ("skewed_train", dict(T=1024, d_model=256, E=8, k=2, d_ff=256, CF=1.0,
                                            zipf_tau=1.0)),
    "bf16_E256_decode_small": ("dsv3_decode", dict(T=64, d_model=512, d_ff=256)),
    # decode-sized segments streamed, K long enough for the two-batch
    # pipeline and its remainder; a shared expert with 48 rows (3 groups)
    "bf16_decode_stream": ("dsv3_decode", dict(T=48, d_model=2048, E=64, E_shared=1, k=4,
                                               d_ff=1024)),
    # the largest k the boundary takes (64 of 128 experts per token) and a
    # shared expert
    "bf16_k64": ("dsv3_decode", dict(T=33, d_model=128, E=128, E_shared=1, k=64, d_ff=128)),
    # T * k < 64 E with T > 64: segments of at most 64 rows stream their
    # weights, larger ones (two experts of 200 and 183 rows and the 200-row
    # shared expert) take the 128-row tiles beside them; twelve experts are
    # empty
    "bf16_decode_mixed_tiles": ("skewed_train", dict(T=200, d_model=256, E=16, E_shared=1, k=2,
                                                     d_ff=256, CF=None, zipf_tau=1.0)),
    # fewer 256 x 256 tiles than compute units and K >= 2048: both phases
    # split K in two and sum the partial tiles
    "bf16_split_k2": ("mixtral_prefill", dict(T=640, d_model=2048, E=4, k=2, d_ff=2048,
                                              CF=1.25)),
    # more tiles than compute units in phase 1: one whole wave of tiles and
    # a split remainder in the same launch
    "bf16_split_mixed": ("mixtral_prefill", dict(T=2048, d_model=2048, E=4, k=2, d_ff=2048,
                                                 CF=1.25)),
    # phase 1 split in four parts (K = 4096), with a shared expert
    "bf16_split_k4_shared": ("dsmoe16b_prefill", dict(T=300, d_model=4096, E=4, E_shared=1,
                                                      k=2, d_ff=1024, CF=1.25)),
    # the smallest dimensions the boundary takes (d = F = 64): the grouped
    # GEMM's K loops run a single 64-wide slice, whose two prologue loads
    # and the loop's last DMA issues all target that slice; H's one column
    # tile holds 64 of its 128 columns
    "bf16_one_slice": ("mixtral_prefill", dict(T=300, d_model=64, E=2, k=1, d_ff=64, CF=None)),
    # F = 192: H's second column tile holds 64 columns (weight rows past F
    # read as zeros, their outputs not stored); d = 320: y's second column
    # tile holds 64 columns
    "bf16_partial_col_tiles": ("mixtral_prefill", dict(T=600, d_model=320, E=2, k=2, d_ff=192,
                                                       CF=None)),
    # the most segments the boundary takes (256 routed + 16 shared): the tile
    # table's per-tile segment search on the 256 x 256 tiles (T k = 64 E:
    # every routed expert a tail tile, 384 tiles) and on the 128-row tiles
    # beside the streaming kernels (T = 100: shared segments of 100 rows)
    "bf16_max_segments_big": ("dsmoe16b_prefill", dict(T=2048, d_model=64, E=256, E_shared=16,
                                                       k=8, d_ff=64, CF=1.25)),
    "bf16_max_segments_mixed": ("dsmoe16b_prefill", dict(T=100, d_model=64, E=256, E_shared=16,
                                                         k=8, d_ff=64, CF=None)),
}


@pytest.mark.parametrize("label", list(SMALL_CASES))
def test_small_layer_matches_oracle(label):
    base, over = SMALL_CASES[label]
    _full_check(get_config(base, **over), label)


def test_all_equal_logits_route_to_the_first_k_and_drop():
    """W_gate = 0: every logit is 0, so every token picks experts 0..k-1 and
    capacity drops all but the first cap tokens of each."""
    import top_routing_expert_softmax_amd as M
    from oracle import moe_oracle as O
    cfg = get_config("mixtral_prefill", T=256, d_model=128, E=8, k=2, d_ff=128, CF=1.0)
    inp = H.LayerInputs(cfg)
    inp.wg[:] = 0.0
    inp.wg_dev.zero_()
    g = H.host(H.run_gpu(inp))
    r, counts, cap, disp, stats = H.oracle_routing(inp)
    assert np.all(g["topk_idx"] == np.arange(2)[None, :])
    H.check_routing(g, r, counts, disp)
    assert g["drop_mask"][:cap].sum() == 0 and g["drop_mask"][cap:].all()
    H.check_stats(g, stats)
    ref = H.oracle_y(inp, r, disp, np.arange(cfg.T))
    H.check_y(cfg, g["y"], ref)
    assert M  # loaded


def test_x_perm_is_exact_copy_and_runs_are_deterministic():
    cfg = get_config("dsmoe16b_prefill", T=512, d_model=256, E=16, E_shared=2, k=4, d_ff=256,
                     CF=1.0)
    inp = H.LayerInputs(cfg)
    b = H.run_gpu(inp)
    R = int(b.offsets[-1].item())
    tor = b.token_of_row[:R].long()
    assert torch.equal(b.x_perm[:R], inp.x_dev[tor])
    # rows of y_perm past R are never written (their contents are undefined)
    outs = {"y_perm": lambda bb: bb.y_perm[:R]}
    for n in ("logits", "topk_idx", "topk_w", "row_of_pair", "y", "y_shared", "f", "P",
              "scalars"):
        outs[n] = lambda bb, n=n: getattr(bb, n)
    first = {n: get(b).clone() for n, get in outs.items()}
    b2 = H.run_gpu(inp, bufs=b)
    for n, get in outs.items():
        assert torch.equal(get(b2), first[n]), f"{n} differs between runs"


FULL = {
    "mixtral_prefill": ("mixtral_prefill", {}),
    "dsv3_decode": ("dsv3_decode", {}),
    "dsmoe16b_prefill": ("dsmoe16b_prefill", {}),
    "skewed_train": ("skewed_train", {}),
    # the DeepSeek-MoE-16B shape (64 routed + 2 shared segments) at capacity
    # factor 1.0, so that its capacity clip drops pairs: at the workload's
    # own CF = 1.25 this seed drops nothing (cap 960, largest count 851)
    "dsmoe16b_prefill_cf1": ("dsmoe16b_prefill", dict(CF=1.0)),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_config(name):
    """Full configuration in the launch configuration the benchmark times:
    routing, permutation and statistics checked in full, and y on every
    token against the oracle's grouped fp64 forward."""
    base, over = FULL[name]
    cfg = get_config(base, **over)
    H.log(f"full config {name}")
    inp = H.LayerInputs(cfg)
    b = H.run_gpu(inp)
    g = H.host(b)
    r, counts, cap, disp, stats = H.oracle_routing(inp)
    H.check_routing(g, r, counts, disp)
    H.check_stats(g, stats)
    R = g["R"]
    tor = b.token_of_row[:R].long()
    assert torch.equal(b.x_perm[:R], inp.x_dev[tor])
    del b
    n_drop = int(disp["drop"].sum())
    if over.get("CF") == 1.0:
        assert n_drop > 0, "this case is meant to drop pairs"
    H.log(f"oracle on all {cfg.T} tokens ({n_drop} dropped pairs)")
    ref = H.oracle_y(inp, r, disp, np.arange(cfg.T))
    mx, mr = H.check_y(cfg, g["y"], ref)
    H.log(f"{name}: R={R} drop={stats['drop_rate']:.4f} max_err={mx:.2e} mean_rel={mr:.2e}")


@pytest.mark.parametrize("d_model,d_ff", [(512, 384), (2048, 1024), (1024, 2048)])
def test_expert_ffn_segments_with_short_remainders(d_model, d_ff):
    """moe_expert_ffn on expert segments of 257, 288, 289, 272, 256, 528 and
    0 rows and a 280-row shared expert: each segment ends in a short row tile
    (1, 32, 33, 16 and 24 rows) or exactly on a 256-row boundary, and an empty
    segment takes no tile.  (2048, 1024) splits phase 1 in K, (1024, 2048)
    phase 2, with short tiles among the split ones.  Every row against the
    oracle's SwiGLU expert; moe_expert_ffn_train gives the same bits and its
    A, B match the oracle."""
    import top_routing_expert_softmax_amd as M
    from oracle import moe_oracle as O
    counts = [257, 288, 289, 272, 256, 528, 0]
    T, k = 280, 7
    cfg = get_config("dsmoe16b_prefill", T=T, d_model=d_model, E=len(counts), E_shared=1, k=k,
                     d_ff=d_ff, CF=None)
    H.log(f"short remainders: {cfg}")
    inp = H.LayerInputs(cfg)
    dd = inp.dev
    R = sum(counts)
    src = np.arange(R) % T                       # x_perm row r copies token r mod T
    xp = torch.zeros((T * k, d_model), dtype=torch.bfloat16, device="cuda")
    xp[:R] = inp.x_dev[torch.from_numpy(src).cuda()]
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32,
                        device="cuda")
    E, F = len(counts), d_ff
    ws = torch.empty(M.moe_workspace_size(T, d_model, E, 1, k, F, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    yp = torch.empty((T * k, d_model), dtype=torch.bfloat16, device="cuda")
    ysh = torch.empty((1, T, d_model), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn(T, k, xp, offs, inp.x_dev, dd["w1"], dd["w3"], dd["w2"], dd["ws1"],
                     dd["ws3"], dd["ws2"], yp, ysh, ws)
    yp2, ysh2 = torch.empty_like(yp), torch.empty_like(ysh)
    ab = torch.empty((T * k + T, 2 * F), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_train(T, k, xp, offs, inp.x_dev, dd["w1"], dd["w3"], dd["w2"], dd["ws1"],
                           dd["ws3"], dd["ws2"], yp2, ysh2, ab, ws)
    torch.cuda.synchronize()
    assert torch.equal(yp[:R], yp2[:R]) and torch.equal(ysh, ysh2)
    x64 = inp.x.astype(np.float64)
    got_y, ref_y, got_ab, ref_ab = [], [], [], []
    o = np.concatenate([[0], np.cumsum(counts)])
    for e in range(E):
        w1, w3, w2 = inp.load_routed(e)
        xr = x64[src[o[e]:o[e + 1]]]
        got_y.append(yp[o[e]:o[e + 1]].float().cpu().numpy())
        ref_y.append(O.swiglu_expert(xr, w1, w3, w2))
        got_ab.append(ab[o[e]:o[e + 1]].float().cpu().numpy())
        ref_ab.append(np.concatenate([xr @ w1.T, xr @ w3.T], axis=1))
    s1, s3, s2 = (a.astype(np.float64) for a in inp.load_shared(0))
    got_y.append(ysh[0].float().cpu().numpy())
    ref_y.append(O.swiglu_expert(x64, s1, s3, s2))
    got_ab.append(ab[T * k:].float().cpu().numpy())
    ref_ab.append(np.concatenate([x64 @ s1.T, x64 @ s3.T], axis=1))
    mx, mr = H.check_y(cfg, np.concatenate(got_y), np.concatenate(ref_y))
    H.log(f"  y: max_err={mx:.2e} mean_rel={mr:.2e}")
    mx, mr = H.check_y(cfg, np.concatenate(got_ab), np.concatenate(ref_ab))
    H.log(f"  A, B: max_err={mx:.2e} mean_rel={mr:.2e}")


def _stream_segments(counts, T, k, d_model, d_ff, E_shared):
    """Explicit segment offsets for the weight-streaming kernels: x_perm row r
    copies token r mod T; every segment of at most 64 rows streams."""
    cfg = get_config("dsv3_decode", T=T, d_model=d_model, E=len(counts), E_shared=E_shared,
                     k=k, d_ff=d_ff, CF=None)
    inp = H.LayerInputs(cfg)
    R = sum(counts)
    src = np.arange(R) % T
    xp = torch.zeros((T * k, d_model), dtype=torch.bfloat16, device="cuda")
    xp[:R] = inp.x_dev[torch.from_numpy(src).cuda()]
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32,
                        device="cuda")
    return cfg, inp, src, xp, offs


@pytest.mark.parametrize("counts,T,k,E_shared", [
    # 1 .. 3 rows read the token rows from LDS (bf16 limit 3), 4 and 5 from
    # L2, 16 and 17 rows one and two token groups, 64 the largest streamed
    ([0, 1, 2, 3, 4, 5, 16, 17, 64, 0, 7], 64, 4, 1),
    # T = 3: the shared expert's all-token segment is staged too
    ([0, 1, 2, 3, 3], 3, 3, 1),
])
def test_stream_segments_at_the_staging_limits(counts, T, k, E_shared):
    """moe_expert_ffn on decode-sized segments with chosen row counts around
    the streaming kernels' LDS staging of token rows, with d = 320 and
    F = 192: rows of 640 and 384 bytes (no whole 1 KB pieces), K loops of 10
    and 6 steps of 32 (whole batches and a remainder).  Every row against
    the oracle's SwiGLU expert."""
    import top_routing_expert_softmax_amd as M
    from oracle import moe_oracle as O
    d_model, d_ff = 320, 192
    cfg, inp, src, xp, offs = _stream_segments(counts, T, k, d_model, d_ff, E_shared)
    H.log(f"stream staging limits: counts={counts} T={T} k={k}")
    dd = inp.dev
    E, F = len(counts), d_ff
    ws = torch.empty(M.moe_workspace_size(T, d_model, E, E_shared, k, F, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    yp = torch.empty((T * k, d_model), dtype=torch.bfloat16, device="cuda")
    ysh = torch.empty((E_shared, T, d_model), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn(T, k, xp, offs, inp.x_dev, dd["w1"], dd["w3"], dd["w2"], dd["ws1"],
                     dd["ws3"], dd["ws2"], yp, ysh, ws)
    torch.cuda.synchronize()
    x64 = inp.x.astype(np.float64)
    o = np.concatenate([[0], np.cumsum(counts)])
    got, ref = [], []
    for e in range(E):
        if counts[e] == 0:
            continue
        w1, w3, w2 = inp.load_routed(e)
        got.append(yp[o[e]:o[e + 1]].float().cpu().numpy())
        ref.append(O.swiglu_expert(x64[src[o[e]:o[e + 1]]], w1, w3, w2))
    s1, s3, s2 = (a.astype(np.float64) for a in inp.load_shared(0))
    got.append(ysh[0].float().cpu().numpy())
    ref.append(O.swiglu_expert(x64, s1, s3, s2))
    mx, mr = H.check_y(cfg, np.concatenate(got), np.concatenate(ref))
    H.log(f"  y: max_err={mx:.2e} mean_rel={mr:.2e}")
