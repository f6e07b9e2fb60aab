"""Pins of the oracle's load-balance statistics, z-loss and drop rate, and of
its routing against the expected-experts-touched closed form."""
import json
import math
import os

import numpy as np

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLDEN, "pages_worked_examples.json")) as fh:
        return json.load(fh)[name]


def test_balance_loss_worked_example():
    g = _gold("balance_example")
    assert math.isclose(O.load_balance_loss(g["f"], g["P"]), g["L"], rel_tol=1e-12)
    E = g["E"]
    assert math.isclose(O.load_balance_loss([1 / E] * E, [1 / E] * E), g["L_balanced"], rel_tol=1e-12)


def test_uniform_routing_gives_E_active():
    for E, k in _gold("uniform_optimum")["cases"]:
        assert math.isclose(O.load_balance_loss([k / E] * E, [1 / E] * E), k, rel_tol=1e-12)


def test_cyclic_logits_reach_the_uniform_optimum_exactly():
    """T = E tokens whose logits are the rotations of one vector c: every
    expert is picked by exactly k tokens and P_i = 1/E, so L = k."""
    rng = np.random.default_rng(0)
    for E, k in [(8, 2), (16, 4), (64, 6)]:
        c = rng.permutation(E).astype(np.float64) * 0.37      # distinct values
        g = np.stack([np.roll(c, t) for t in range(E)])
        idx = O.topk_experts(g, k)
        counts = O.expert_counts(idx, E)
        assert np.all(counts == k)
        s = O.aux_stats(g, counts, E, k, cap=E)
        assert np.allclose(s["f"], k / E, rtol=0, atol=0)
        assert np.allclose(s["P"], 1.0 / E, rtol=1e-14)
        assert math.isclose(s["L_balance"], k, rel_tol=1e-13)


def test_equal_logits_give_P_uniform_and_L_equal_k():
    T, E, k = 10, 16, 4
    g = np.full((T, E), 0.5)
    idx = O.topk_experts(g, k)
    counts = O.expert_counts(idx, E)
    s = O.aux_stats(g, counts, T, k, cap=T)
    assert np.allclose(s["P"], 1 / E, rtol=1e-15)
    assert math.isclose(s["L_balance"], k, rel_tol=1e-14)


def test_f_sums_to_k():
    rng = np.random.default_rng(1)
    for T, E, k in [(100, 8, 2), (77, 64, 6), (64, 256, 8)]:
        g = rng.normal(size=(T, E))
        counts = O.expert_counts(O.topk_experts(g, k), E)
        s = O.aux_stats(g, counts, T, k, cap=T)
        assert math.isclose(s["f"].sum(), k, rel_tol=1e-14)
        assert math.isclose(s["P"].sum(), 1.0, rel_tol=1e-13)


def test_z_loss_closed_forms():
    T = 5
    for E, c in [(256, 0.0), (8, 1.5), (16, -2.0)]:
        g = np.full((T, E), c)
        counts = O.expert_counts(O.topk_experts(g, 2), E)
        s = O.aux_stats(g, counts, T, 2, cap=T)
        assert math.isclose(s["z_loss"], (c + math.log(E)) ** 2, rel_tol=1e-14)
    # E=256, c=0: (ln 256)^2
    assert math.isclose(math.log(256) ** 2, 30.7488, rel_tol=1e-5)
    # shifting a row by c shifts its lse by c
    rng = np.random.default_rng(2)
    g = rng.normal(size=(7, 16))
    assert np.allclose(O.logsumexp(g + 3.25), O.logsumexp(g) + 3.25, rtol=1e-14)


def test_drop_rate_counts_pairs_over_capacity():
    rng = np.random.default_rng(3)
    T, E, k = 200, 8, 2
    g = rng.normal(size=(T, E))
    g[:, 2] += 1.5
    idx = O.topk_experts(g, k)
    counts = O.expert_counts(idx, E)
    cap = O.capacity(T, E, k, 1.0)
    d = O.dispatch(idx, E, cap)
    s = O.aux_stats(g, counts, T, k, cap)
    assert d["drop"].sum() > 0
    assert math.isclose(s["drop_rate"], d["drop"].sum() / (T * k), rel_tol=1e-15)


def test_hand_worked_stats_example():
    with open(os.path.join(GOLDEN, "tiny_routing_hand.json")) as fh:
        h = json.load(fh)
    g = np.array(h["logits"])
    s = O.aux_stats(g, h["counts"], len(g), h["k"], h["capacity"])
    assert np.allclose(s["f"], h["f"], rtol=1e-15)
    assert s["drop_rate"] == h["drop_rate"]


def test_expected_experts_touched_closed_form():
    """With exchangeable logits each expert is in a token's top-k with
    probability k/E, so B independent tokens touch E(1-(1-k/E)^B) experts in
    expectation.  Monte Carlo through the oracle's top-k, within 4 standard
    errors, and the closed form against the printed values."""
    rng = np.random.default_rng(4)
    for case in _gold("experts_touched")["cases"]:
        E, k, B = case["E"], case["k"], case["B"]
        closed = E * (1 - (1 - k / E) ** B)
        assert round(closed, case["printed_digits"]) == case["printed"]
        trials = 1500
        touched = np.empty(trials)
        for i in range(trials):
            idx = O.topk_experts(rng.normal(size=(B, E)), k)
            touched[i] = len(np.unique(idx))
        se = touched.std(ddof=1) / math.sqrt(trials)
        assert abs(touched.mean() - closed) < 4 * se + 1e-9, (touched.mean(), closed, se)
