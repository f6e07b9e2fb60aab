"""The seeded generator: grid exactness, bf16 rounding, determinism, and the
skewed workload's drop rate staying in the band the pages give for CF=1.0."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from workloads import (CONFIGS, bf16_bits_to_f32, expert_weight, f32_to_bf16_bits,
                       get_config, router_inputs)


def test_bf16_rounding_is_round_to_nearest_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even (1.0)
    a = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0], np.float32)
    back = bf16_bits_to_f32(f32_to_bf16_bits(a))
    assert back.tolist() == [1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0]
    # agrees with torch's own conversion
    import torch
    rng = np.random.default_rng(0)
    v = rng.normal(size=10000).astype(np.float32)
    t = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(v)), t)


@pytest.mark.parametrize("name", ["tiny_f32", "mixtral_prefill", "dsv3_decode", "dsmoe16b_prefill"])
def test_router_grid_bound_holds(name):
    cfg = CONFIGS[name]
    if cfg.T > 1024:
        cfg = get_config(name, T=1024)
    x, wg = router_inputs(cfg, check_grid=True)   # raises if violated
    assert x.dtype == np.float32 and wg.dtype == np.float32


def test_generation_is_deterministic_and_per_expert():
    cfg = get_config("dsmoe16b_prefill", T=16)
    a = expert_weight(cfg, "w1", 3)
    b = expert_weight(cfg, "w1", 3)
    c = expert_weight(cfg, "w1", 4)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert a.shape == (cfg.d_ff, cfg.d_model)
    assert abs(float(a.std()) - 0.02) < 0.001


def test_skewed_workload_drop_rate_in_band():
    """'MoE routing math' section 4.3: CF = 1.0 drops 5-15% of pairs."""
    cfg = CONFIGS["skewed_train"]
    x, wg = router_inputs(cfg)
    g = O.router_logits(x, wg)
    counts = O.expert_counts(O.topk_experts(g, cfg.k), cfg.E)
    cap = O.capacity(cfg.T, cfg.E, cfg.k, cfg.CF)
    rate = np.maximum(counts - cap, 0).sum() / (cfg.T * cfg.k)
    assert 0.05 <= rate <= 0.15, rate
