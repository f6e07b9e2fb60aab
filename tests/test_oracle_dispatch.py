"""Pins of the oracle's counting, capacity, drop and permutation."""
import json
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from workloads import CONFIGS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLDEN, "pages_worked_examples.json")) as fh:
        return json.load(fh)[name]


def _random_routing(T, E, k, rng, skew=0.0):
    g = rng.normal(size=(T, E))
    g[:, 0] += skew
    return O.topk_experts(g, k)


def test_capacity_worked_example():
    c = _gold("capacity_example")
    assert O.capacity(c["n_tokens"], c["E"], c["k"], c["cf"]) == c["capacity"]


def test_capacity_of_the_configs():
    want = {"tiny_f32": 20, "mixtral_prefill": 4096, "dsv3_decode": 64,
            "dsmoe16b_prefill": 960, "skewed_train": 4096}
    for name, cap in want.items():
        c = CONFIGS[name]
        assert O.capacity(c.T, c.E, c.k, c.CF) == cap


def test_capacity_rounds_up_and_clamps():
    assert O.capacity(3, 4, 2, 0.5) == 1        # ceil(0.75)
    assert O.capacity(10, 3, 1, 1.0) == 4       # ceil(10/3)
    assert O.capacity(12, 3, 1, 1.0) == 4       # exact, no rounding up
    assert O.capacity(100, 2, 2, 5.0) == 100    # clamped to T
    assert O.capacity(100, 8, 2, None) == 100   # no limit
    assert O.capacity(100, 8, 2, 0.0) == 100


def test_worked_example_drops_exactly_the_last_80():
    """2048 tokens, 16 experts, k=2, cf=1.25: an expert picked 400 times keeps
    its first 320 tokens and drops the last 80."""
    c = _gold("capacity_example")
    T, E, k = c["n_tokens"], c["E"], c["k"]
    rng = np.random.default_rng(5)
    idx = np.zeros((T, k), dtype=np.int64)
    hot = np.sort(rng.choice(T, size=c["times_chosen"], replace=False))
    for t in range(T):
        others = rng.choice(np.arange(1, E), size=2, replace=False)
        if t in set(hot.tolist()):
            idx[t] = [0, others[0]]
        else:
            idx[t] = others
    # keep the other experts under capacity so only expert 0 overflows
    cap = O.capacity(T, E, k, c["cf"])
    counts = O.expert_counts(idx, E)
    assert counts[0] == c["times_chosen"] and counts[1:].max() <= cap
    d = O.dispatch(idx, E, cap)
    dropped_tokens = np.nonzero(d["drop"][:, 0])[0]
    assert len(dropped_tokens) == c["dropped"]
    assert np.array_equal(dropped_tokens, hot[-c["dropped"]:])
    assert int(d["drop"].sum()) == c["dropped"]


def test_counts_bruteforce_and_sum():
    rng = np.random.default_rng(1)
    for T, E, k in [(1, 4, 1), (7, 8, 2), (64, 16, 4), (33, 256, 8)]:
        idx = _random_routing(T, E, k, rng)
        counts = O.expert_counts(idx, E)
        brute = [sum(1 for t in range(T) for j in range(k) if idx[t, j] == e) for e in range(E)]
        assert counts.tolist() == brute
        assert counts.sum() == T * k


@pytest.mark.parametrize("skew", [0.0, 1.5, 4.0])
def test_dispatch_invariants(skew):
    rng = np.random.default_rng(2)
    T, E, k = 300, 8, 2
    idx = _random_routing(T, E, k, rng, skew)
    cap = O.capacity(T, E, k, 1.0)
    counts = O.expert_counts(idx, E)
    d = O.dispatch(idx, E, cap)
    # kept_e = min(counts_e, cap)
    assert np.array_equal(d["kept"], np.minimum(counts, cap))
    # per expert, kept tokens precede dropped ones in token order
    for e in range(E):
        toks = [(t, int(d["drop"][t, j])) for t in range(T) for j in range(k) if idx[t, j] == e]
        flags = [f for _, f in toks]
        assert flags == sorted(flags)
        assert sum(flags) == max(0, counts[e] - cap)
    # rows: a bijection between kept pairs and [0, R), sorted by (expert, token)
    R = int(d["offsets"][-1])
    rows = d["row_of_pair"][d["drop"] == 0]
    assert sorted(rows.tolist()) == list(range(R))
    keys = []
    for r in range(R):
        t = int(d["token_of_row"][r])
        j = int(np.nonzero(d["row_of_pair"][t] == r)[0][0])
        keys.append((int(idx[t, j]), t))
    assert keys == sorted(keys)
    assert np.all(d["token_of_row"][R:] == -1)
    # offsets bracket each expert's rows
    for e in range(E):
        for r in range(d["offsets"][e], d["offsets"][e + 1]):
            t = int(d["token_of_row"][r])
            assert e in idx[t]


def test_no_capacity_means_no_drop():
    rng = np.random.default_rng(3)
    idx = _random_routing(64, 256, 8, rng)
    d = O.dispatch(idx, 256, O.capacity(64, 256, 8, None))
    assert d["drop"].sum() == 0 and d["offsets"][-1] == 64 * 8


def test_every_token_to_one_expert():
    """All tokens pick expert 0 first: it keeps exactly cap of them."""
    T, E, k = 50, 4, 2
    idx = np.stack([np.zeros(T, dtype=np.int64), 1 + (np.arange(T) % 3)], axis=1)
    cap = O.capacity(T, E, k, 1.0)           # ceil(25) = 25
    d = O.dispatch(idx, E, cap)
    assert d["kept"][0] == cap == 25
    assert d["drop"][:, 0].tolist() == [0] * 25 + [1] * 25
    assert d["drop"][:, 1].sum() == 0


def test_hand_worked_dispatch_example():
    with open(os.path.join(GOLDEN, "tiny_routing_hand.json")) as fh:
        h = json.load(fh)
    idx = np.array(h["idx"])
    T = idx.shape[0]
    cap = O.capacity(T, h["E"], h["k"], h["cf"])
    assert cap == h["capacity"]
    assert O.expert_counts(idx, h["E"]).tolist() == h["counts"]
    d = O.dispatch(idx, h["E"], cap)
    for key in ("drop", "kept", "offsets", "row_of_pair", "token_of_row"):
        assert d[key].tolist() == h[key], key
