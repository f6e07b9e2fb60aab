"""Pins of the DeepSeek-V3 gate in the oracle ("CMU 11-868 Lecture 17",
sections 3.4, 4.3 and 5.3): hand-worked examples, the fixed weight sum, the
group limit, the page's distinct-group counts, the reduction to a plain
top-k, and that the bias moves only the choice."""
import json
import math
import os

import numpy as np
import pytest

from oracle import moe_oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "v3_gate_hand.json")))


def test_group_score_is_the_sum_of_the_two_largest():
    c = GOLD["groups_by_top2"]
    g = np.array([c["logits"]], dtype=np.float64)
    r = O.v3_gate(g, c["bias"], c["k"], c["n_groups"], c["topk_groups"], c["route_scale"])
    np.testing.assert_allclose(r["biased"][0], c["biased_hand"], rtol=0, atol=1e-6)
    np.testing.assert_allclose(r["group_score"][0], c["group_score_hand"], rtol=0, atol=1e-6)
    assert r["idx"][0].tolist() == c["idx"]
    np.testing.assert_allclose(r["weights"][0], c["weights"], rtol=1e-12)


def test_ties_go_low_and_weights_use_unbiased_affinities():
    c = GOLD["ties_and_affinities"]
    g = np.array([c["logits_ln3"]], dtype=np.float64) * math.log(3.0)
    r = O.v3_gate(g, c["bias"], c["k"], c["n_groups"], c["topk_groups"], c["route_scale"])
    assert r["affinity"][0].tolist() == [0.75, 0.5, 0.5, 0.25, 0.5, 0.5, 0.5, 0.5]
    np.testing.assert_allclose(r["biased"][0], c["biased_hand"], rtol=0, atol=1e-6)
    np.testing.assert_allclose(r["group_score"][0], c["group_score_hand"], rtol=0, atol=1e-6)
    assert r["kept_groups"][0].tolist() == c["kept_groups"]
    assert r["idx"][0].tolist() == c["idx"]
    np.testing.assert_allclose(r["weights"][0], c["weights"], rtol=1e-12)


def test_bias_step():
    c = GOLD["bias_step"]
    b = O.update_bias(c["counts"], c["bias"], c["T"], c["k"], c["gamma"])
    assert b.dtype == np.float32
    np.testing.assert_array_equal(b, np.array(c["bias_after"], dtype=np.float32))


def test_weights_sum_to_route_scale_and_groups_are_limited():
    """L17 section 5.3: the weights of a token always sum to 2.5, and its 8
    experts come from at most 4 groups."""
    rng = np.random.default_rng(1)
    g = rng.standard_normal((512, 256))
    b = rng.uniform(-0.1, 0.1, 256)
    r = O.v3_gate(g, b, 8, 8, 4, 2.5)
    np.testing.assert_allclose(r["weights"].sum(axis=1), 2.5, rtol=1e-13)
    groups = r["idx"] // 32
    assert max(len(set(row.tolist())) for row in groups) <= 4
    # every chosen expert lies in a kept group, and is among the k best there
    for t in range(0, 512, 37):
        kept = set(r["kept_groups"][t].tolist())
        assert set((r["idx"][t] // 32).tolist()) <= kept
        allowed = [e for e in range(256) if e // 32 in kept]
        best = sorted(allowed, key=lambda e: (-float(r["biased"][t, e]), e))[:8]
        assert r["idx"][t].tolist() == best


def test_distinct_groups_match_the_page():
    """L17 section 4.3: with random scores a token's 8 experts span 5.30
    groups on average without the limit and 3.96 with 4 groups kept.  The
    first is also 8 (1 - C(224, 8) / C(256, 8)) = 5.2947 in closed form
    (iid scores make every 8-subset equally likely).  Tolerances: 4
    standard errors of this estimate, plus, against the page's own 2000-token
    estimate, half a unit of its last digit and 4 of its standard errors."""
    rng = np.random.default_rng(7)
    T = 20000
    g = rng.standard_normal((T, 256))
    out = {}
    for tg in (8, 4):
        r = O.v3_gate(g, np.zeros(256), 8, 8, tg, 2.5)
        ng = np.array([len(set(row.tolist())) for row in (r["idx"] // 32)])
        out[tg] = (ng.mean(), ng.std() / math.sqrt(T), ng.std())
    closed = 8 * (1 - math.prod((224 - i) / (256 - i) for i in range(8)))
    m8, se8, sd8 = out[8]
    assert abs(m8 - closed) < 4 * se8
    assert abs(m8 - 5.30) < 0.005 + 4 * sd8 / math.sqrt(2000) + 4 * se8
    m4, se4, sd4 = out[4]
    assert abs(m4 - 3.96) < 0.005 + 4 * sd4 / math.sqrt(2000) + 4 * se4


def test_without_groups_or_bias_it_is_the_plain_top_k():
    """One group (or all groups kept) and zero bias: sigmoid is increasing,
    so the choice is the top-k of the logits, the same ids as the softmax
    router's (RM section 2.1)."""
    rng = np.random.default_rng(3)
    g = rng.integers(-500, 500, size=(300, 64)) / 64.0
    want = O.topk_experts(g, 6)
    for n_groups, tg in ((1, 1), (8, 8), (16, 16)):
        r = O.v3_gate(g, np.zeros(64), 6, n_groups, tg, 1.0)
        np.testing.assert_array_equal(r["idx"], want)
        s = 1.0 / (1.0 + np.exp(-g))
        sel = np.take_along_axis(s, want, axis=1)
        np.testing.assert_allclose(r["weights"], sel / sel.sum(axis=1, keepdims=True),
                                   rtol=1e-6)


def test_bias_moves_only_the_choice():
    """L17 section 5.3, third property: raising one expert's bias by 0.3
    makes far more tokens choose it, while tokens whose chosen set did not
    change keep their weights exactly."""
    rng = np.random.default_rng(5)
    g = rng.standard_normal((2000, 256))
    b = np.zeros(256)
    r0 = O.v3_gate(g, b, 8, 8, 4, 2.5)
    b1 = b.copy()
    b1[17] += 0.3
    r1 = O.v3_gate(g, b1, 8, 8, 4, 2.5)
    n0 = int((r0["idx"] == 17).any(axis=1).sum())
    n1 = int((r1["idx"] == 17).any(axis=1).sum())
    assert n1 > 5 * max(n0, 1)
    same = [t for t in range(2000) if sorted(r0["idx"][t]) == sorted(r1["idx"][t])]
    assert len(same) > 100
    for t in same:
        w0 = dict(zip(r0["idx"][t].tolist(), r0["weights"][t].tolist()))
        w1 = dict(zip(r1["idx"][t].tolist(), r1["weights"][t].tolist()))
        assert w0 == w1


def test_bad_groups_are_rejected():
    with pytest.raises(ValueError):
        O.v3_gate(np.zeros((1, 10)), np.zeros(10), 2, 3, 1, 1.0)
    with pytest.raises(ValueError):
        O.v3_gate(np.zeros((1, 8)), np.zeros(8), 2, 8, 1, 1.0)
