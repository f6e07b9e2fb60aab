"""The five seeded workloads of the MoE-layer forward.

Shapes follow the models the pages name: a tiny fp32 layer, a Mixtral-8x7B
layer (E=8, k=2, d_ff=14336; "MoE routing math" section 1 table, and the CMU
11-868 lecture 17 notes section 1.2), a DeepSeek-V3 decode step (E=256 routed +
1 shared, k=8, d_ff=2048, d=7168; lecture 17 notes section 5.2), a
DeepSeekMoE-16B layer (E=64, k=6; "MoE routing math" section 1 table) and a
skewed training-style forward (E=16, k=4, Zipf-ranked expert offsets).

Router recipe (the dyadic grid): x = m * 2**-4 with integer m, and
W_gate = n * 2**-wg_shift with integer |n| <= 255, so every value is exact in
bf16 and every fp32 partial sum of x.W_gate is exact as long as
sum_i |m_i * n_i| < 2**24 for every (token, expert); the generator checks that
bound.
"""
from dataclasses import dataclass, field
from typing import Optional


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens
    d_model: int           # hidden size d
    E: int                 # routed experts
    E_shared: int          # always-on shared experts
    k: int                 # experts chosen per token (E_active)
    d_ff: int              # expert intermediate size F
    CF: Optional[float]    # capacity factor; None means no capacity limit
    dtype: str             # "f32" or "bf16": activations and weights
    seed: int              # master seed
    x_kind: str            # "uniform16": m ~ U{-8..8}; "gauss16": m = clip(round(16 z), +-128)
    wg_shift: int          # W_gate = n * 2**-wg_shift
    wg_kind: str           # "uniform": n ~ U{-8..8}; "gauss": n = clip(round(N(0, wg_sd^2)), +-255)
    wg_sd: float = 0.0
    zipf_s: float = 0.0    # > 0: x[:,0] = 1 and W_gate[0,:] holds Zipf-ranked offsets
    zipf_tau: float = 0.0  # temperature of those offsets (oracle/calibrate_zipf.py picks it)
    w_sd: float = 0.02     # expert weights ~ N(0, w_sd^2)
    note: str = field(default="", compare=False)

    @property
    def bytes_per_el(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS = {
    "tiny_f32": MoEConfig(
        name="tiny_f32", T=64, d_model=128, E=8, E_shared=0, k=2, d_ff=256,
        CF=1.25, dtype="f32", seed=1, x_kind="uniform16", wg_shift=4,
        wg_kind="uniform",
        note="tiny fp32 layer: overflow dropped in token order (cap 20 vs mean 16)"),
    "mixtral_prefill": MoEConfig(
        name="mixtral_prefill", T=4096, d_model=4096, E=8, E_shared=0, k=2,
        d_ff=14336, CF=4.0, dtype="bf16", seed=2, x_kind="gauss16",
        wg_shift=11, wg_kind="gauss", wg_sd=32.0,
        note="Mixtral-shaped prefill, CF = E/k so nothing is dropped"),
    "dsv3_decode": MoEConfig(
        name="dsv3_decode", T=64, d_model=7168, E=256, E_shared=1, k=8,
        d_ff=2048, CF=None, dtype="bf16", seed=3, x_kind="gauss16",
        wg_shift=14, wg_kind="gauss", wg_sd=20.0,
        note="DeepSeek-V3-shaped decode step, near-uniform logits, no drop"),
    "dsmoe16b_prefill": MoEConfig(
        name="dsmoe16b_prefill", T=8192, d_model=2048, E=64, E_shared=2, k=6,
        d_ff=1408, CF=1.25, dtype="bf16", seed=4, x_kind="gauss16",
        wg_shift=11, wg_kind="gauss", wg_sd=45.0,
        note="DeepSeekMoE-16B-shaped prefill, CF 1.25 with drop"),
    "skewed_train": MoEConfig(
        name="skewed_train", T=16384, d_model=4096, E=16, E_shared=0, k=4,
        d_ff=10752, CF=1.0, dtype="bf16", seed=5, x_kind="gauss16",
        wg_shift=11, wg_kind="gauss", wg_sd=32.0, zipf_s=1.2, zipf_tau=0.2,
        note="skewed training-style forward, Zipf(1.2)-ranked offsets, CF 1.0"),
}

ORDER = ["tiny_f32", "mixtral_prefill", "dsv3_decode", "dsmoe16b_prefill",
         "skewed_train"]


def get_config(name: str, **overrides) -> MoEConfig:
    """Config by name; keyword overrides give a reduced copy (same recipe)."""
    base = CONFIGS[name]
    if not overrides:
        return base
    d = dict(base.__dict__)
    d.update(overrides)
    return MoEConfig(**d)
