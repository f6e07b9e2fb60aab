"""Pins of the oracle's router (logits, softmax, top-k, renormalisation).

Each check is fixed by something other than the oracle's own formula: integer
arithmetic, brute force over all subsets, closed forms, or a hand-worked case.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import moe_oracle as O
from workloads import get_config, router_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_topk(g_row, k):
    """The unique k-subset S such that each member beats each non-member under
    (larger logit, then lower index); returned in that order."""
    E = len(g_row)

    def beats(i, j):
        return g_row[i] > g_row[j] or (g_row[i] == g_row[j] and i < j)

    found = []
    for S in itertools.combinations(range(E), k):
        rest = [j for j in range(E) if j not in S]
        if all(beats(i, j) for i in S for j in rest):
            found.append(S)
    assert len(found) == 1
    S = list(found[0])
    # order inside S by the same relation (insertion sort by "beats")
    out = []
    for i in S:
        pos = 0
        while pos < len(out) and beats(out[pos], i):
            pos += 1
        out.insert(pos, i)
    return out


def test_logits_exact_integer_tiny():
    """x.W_gate on the dyadic grid equals the integer dot product, exactly."""
    cfg = get_config("tiny_f32")
    x, wg = router_inputs(cfg)
    g = O.router_logits(x, wg)
    m = np.rint(x.astype(np.float64) * 16).astype(np.int64)
    n = np.rint(wg.astype(np.float64) * 2 ** cfg.wg_shift).astype(np.int64)
    for t in range(cfg.T):
        for e in range(cfg.E):
            s = sum(int(m[t, i]) * int(n[i, e]) for i in range(cfg.d_model))
            assert Fraction(float(g[t, e])) == Fraction(s, 2 ** (4 + cfg.wg_shift))


@pytest.mark.parametrize("name", ["mixtral_prefill", "dsv3_decode", "skewed_train"])
def test_logits_exact_integer_sampled_rows(name):
    """Sampled rows of the large configs, also against integer arithmetic."""
    cfg = get_config(name)
    cfg = get_config(name, T=64) if cfg.T > 64 else cfg
    x, wg = router_inputs(cfg)
    g = O.router_logits(x, wg)
    m = np.rint(x.astype(np.float64) * 16).astype(object)
    n = np.rint(wg.astype(np.float64) * 2 ** cfg.wg_shift).astype(object)
    rows = [0, 1, 17, cfg.T - 1]
    exact = m[rows] @ n          # Python ints, no rounding anywhere
    for a, t in enumerate(rows):
        for e in range(cfg.E):
            assert Fraction(float(g[t, e])) == Fraction(int(exact[a, e]), 2 ** (4 + cfg.wg_shift))


def test_topk_bruteforce_small_with_ties():
    rng = np.random.default_rng(7)
    for E in (2, 3, 5, 8):
        for k in range(1, min(E, 4) + 1):
            for _ in range(40):
                g = rng.integers(-3, 4, size=E).astype(np.float64)  # many ties
                got = list(O.topk_experts(g[None, :], k)[0])
                assert got == _brute_topk(list(g), k)


def test_topk_on_probabilities_equals_topk_on_logits():
    """Softmax is strictly increasing, so TopK(p) and TopK(g) coincide
    (also in fp64 on the grid: distinct grid logits give distinct p)."""
    cfg = get_config("tiny_f32")
    x, wg = router_inputs(cfg)
    g = O.router_logits(x, wg)
    assert np.array_equal(O.topk_experts(O.softmax(g), cfg.k), O.topk_experts(g, cfg.k))


def test_topk_all_equal_logits():
    for E, k in [(8, 2), (16, 4), (256, 8)]:
        g = np.zeros((3, E))
        assert np.array_equal(O.topk_experts(g, k), np.tile(np.arange(k), (3, 1)))


def test_renormalised_weights_sum_to_one():
    with open(os.path.join(GOLDEN, "pages_worked_examples.json")) as fh:
        gold = json.load(fh)["weight_sums"]
    rng = np.random.default_rng(3)
    g = rng.normal(size=(200, 16)) * 3
    p = O.softmax(g)
    for k in (1, 2, 4, 8):
        w = O.renormalise(p, O.topk_experts(p, k))
        assert np.allclose(w.sum(axis=1), gold["sum"], rtol=0, atol=1e-15)
        assert np.all(w > 0)


def test_two_forms_give_the_same_weights():
    """softmax -> TopK -> renormalise equals TopK on logits -> softmax of the k
    values (the pages give both forms)."""
    rng = np.random.default_rng(11)
    for E, k in [(8, 2), (64, 6), (16, 4), (256, 8)]:
        g = rng.normal(size=(100, E)) * 2
        p = O.softmax(g)
        idx_a = O.topk_experts(p, k)
        w_a = O.renormalise(p, idx_a)
        idx_b, w_b = O.topk_softmax_weights(g, k)
        assert np.array_equal(idx_a, idx_b)
        assert np.allclose(w_a, w_b, rtol=1e-13, atol=0)


def test_equal_top_logits_give_uniform_weights():
    g = np.array([[5.0, 5.0, 5.0, 1.0, -2.0, 5.0]])
    idx = O.topk_experts(O.softmax(g), 4)
    assert list(idx[0]) == [0, 1, 2, 5]
    assert np.allclose(O.renormalise(O.softmax(g), idx), 0.25, atol=1e-16)


def test_softmax_and_lse_closed_forms():
    # two experts: p = sigmoid(g0 - g1)
    g = np.array([[0.3, -1.2]])
    assert math.isclose(O.softmax(g)[0, 0], 1 / (1 + math.exp(-1.5)), rel_tol=1e-15)
    # lse of equal logits c over E experts is c + ln E
    assert math.isclose(O.logsumexp(np.full((1, 256), 0.0))[0], math.log(256), rel_tol=1e-15)
    assert math.isclose(O.logsumexp(np.full((1, 8), 7.0))[0], 7.0 + math.log(8), rel_tol=1e-15)


def test_hand_worked_routing_example():
    with open(os.path.join(GOLDEN, "tiny_routing_hand.json")) as fh:
        h = json.load(fh)
    g = np.array(h["logits"])
    r_idx = O.topk_experts(O.softmax(g), h["k"])
    assert r_idx.tolist() == h["idx"]
    w = O.renormalise(O.softmax(g), r_idx)
    e2 = math.exp(2.0)
    want = np.array([[0.5, 0.5], [0.5, 0.5], [e2 / (e2 + 1), 1 / (e2 + 1)]])
    assert np.allclose(w, want, rtol=1e-15, atol=0)
