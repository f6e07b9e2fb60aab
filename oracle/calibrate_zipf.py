"""Choose the temperature of the skewed workload's Zipf offsets.

TEST INFRASTRUCTURE: calls only the oracle and the input generator.  For each
tau on a fixed grid it routes the full skewed batch (T=16384, E=16, k=4,
CF=1.0) with the oracle and prints the drop rate; the chosen tau is the grid
value whose drop rate is closest to 10%, the middle of the 5-15% band that
"MoE routing math" section 4.3 gives for CF = 1.0.

    python -m oracle.calibrate_zipf
"""
import numpy as np

from oracle import moe_oracle as O
from workloads import get_config, router_inputs

GRID = (0.2, 0.4, 0.6, 0.8, 1.0)


def drop_rate(tau: float) -> float:
    cfg = get_config("skewed_train", zipf_tau=tau)
    x, wg = router_inputs(cfg)
    g = O.router_logits(x, wg)
    idx = O.topk_experts(g, cfg.k)
    counts = O.expert_counts(idx, cfg.E)
    cap = O.capacity(cfg.T, cfg.E, cfg.k, cfg.CF)
    return float(np.maximum(counts - cap, 0).sum()) / (cfg.T * cfg.k)


def main():
    rates = {tau: drop_rate(tau) for tau in GRID}
    for tau, r in rates.items():
        print(f"tau={tau:.1f} drop_rate={r:.4f}")
    best = min(GRID, key=lambda t: abs(rates[t] - 0.10))
    print(f"chosen tau={best}")


if __name__ == "__main__":
    main()
