"""Pins of expert-choice routing in the oracle ("MoE deep dive: routing
mechanisms and load balancing", section 2.2): a hand-worked example, the
capacity rule, perfect balance, brute force on small inputs, and the E = 1
case that reduces to a dense SwiGLU FFN."""
import itertools
import json
import os

import numpy as np

from oracle import moe_oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "expert_choice_hand.json")))


def test_hand_example():
    c = GOLD
    assert O.ec_capacity(c["T"], c["E"], c["cf"]) == c["capacity"]
    r = O.expert_choice(np.array(c["logits"]), c["capacity"])
    assert r["tokens"].tolist() == c["tokens"]
    chosen = np.bincount(r["tokens"].ravel(), minlength=c["T"])
    assert chosen.tolist() == c["times_chosen"]
    assert [t for t in range(c["T"]) if chosen[t] == 0] == c["unchosen_tokens"]
    p = O.softmax(np.array(c["logits"]))
    for e in range(c["E"]):
        np.testing.assert_allclose(r["weights"][e], p[r["tokens"][e], e], rtol=1e-15)


def test_capacity_rule():
    for T, E, cf, want in GOLD["capacity_cases"]:
        assert O.ec_capacity(T, E, cf) == want, (T, E, cf)


def test_every_expert_takes_exactly_cap_tokens_and_brute_force():
    """Balance by construction, and on small inputs the chosen set of each
    expert is the unique cap-subset whose logits beat every unchosen one
    (equal logits: the lower token wins)."""
    rng = np.random.default_rng(0)
    for _ in range(40):
        T = int(rng.integers(2, 9))
        E = int(rng.integers(1, 4))
        g = rng.integers(-3, 4, size=(T, E)).astype(np.float64)   # many ties
        cap = O.ec_capacity(T, E, float(rng.choice([1.0, 1.5, 2.0])))
        r = O.expert_choice(g, cap)
        assert r["tokens"].shape == (E, cap)
        for e in range(E):
            col = g[:, e]
            good = []
            for S in itertools.combinations(range(T), cap):
                out = [t for t in range(T) if t not in S]
                if all(col[i] > col[j] or (col[i] == col[j] and i < j) for i in S for j in out):
                    good.append(S)
            assert len(good) == 1
            assert sorted(r["tokens"][e].tolist()) == list(good[0])
            # order: larger logit first, ties to the lower token
            seq = r["tokens"][e].tolist()
            keys = [(-col[t], t) for t in seq]
            assert keys == sorted(keys)


def test_single_expert_is_a_dense_ffn():
    """E = 1, CF = 1: the expert takes every token, each with probability
    1, so the layer is the dense SwiGLU MLP (numpy, written out)."""
    rng = np.random.default_rng(1)
    T, d, F = 12, 8, 16
    x = rng.standard_normal((T, d))
    g = rng.standard_normal((T, 1))
    w1 = rng.standard_normal((F, d)); w3 = rng.standard_normal((F, d))
    w2 = rng.standard_normal((d, F))
    cap = O.ec_capacity(T, 1, 1.0)
    r = O.expert_choice(g, cap)
    assert sorted(r["tokens"][0].tolist()) == list(range(T))
    np.testing.assert_allclose(r["weights"], 1.0)
    y = O.ec_combine(x, r["tokens"], r["weights"], lambda e: (w1, w3, w2))
    h = x @ w1.T
    dense = ((h / (1 + np.exp(-h))) * (x @ w3.T)) @ w2.T
    np.testing.assert_allclose(y, dense, rtol=1e-12, atol=1e-12)


def test_dispatch_maps_are_inverse():
    rng = np.random.default_rng(2)
    T, E = 50, 5
    g = rng.standard_normal((T, E))
    cap = O.ec_capacity(T, E, 2.0)
    r = O.expert_choice(g, cap)
    dsp = O.ec_dispatch(r["tokens"], r["weights"], T)
    assert dsp["offsets"].tolist() == [e * cap for e in range(E + 1)]
    for t in range(T):
        for e in range(E):
            row = dsp["row_of_te"][t, e]
            if row >= 0:
                assert dsp["token_of_row"][row] == t and row // cap == e
                assert dsp["w_te"][t, e] == r["weights"][e, row % cap]
            else:
                assert t not in r["tokens"][e] and dsp["w_te"][t, e] == 0
