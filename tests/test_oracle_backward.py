"""Pins of the oracle's backward pass: central finite differences of the
loss L = sum(dy * y) + alpha L_balance + beta z on small layers (drops,
shared experts, all parameter kinds), and the one-expert dense SwiGLU MLP
against torch's autograd."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def _loss(x, wg, experts, shared, k, CF, dy, alpha, beta):
    E = wg.shape[1]
    out = O.layer_forward(x, wg, k, CF, lambda e: experts[e], E, len(shared),
                          (lambda s: shared[s]) if shared else None)
    return float(np.sum(dy * out["y"]) + alpha * out["L_balance"] + beta * out["z_loss"]), out


def _setup(seed, T=7, d=5, E=4, k=2, F=6, n_shared=1):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((d, E))
    experts = [tuple(rng.standard_normal(s) * 0.5 for s in ((F, d), (F, d), (d, F)))
               for _ in range(E)]
    shared = [tuple(rng.standard_normal(s) * 0.5 for s in ((F, d), (F, d), (d, F)))
              for _ in range(n_shared)]
    dy = rng.standard_normal((T, d))
    return x, wg, experts, shared, dy


@pytest.mark.parametrize("seed,CF", [(0, 0.75), (1, None), (2, 0.5)])
def test_gradients_match_central_differences(seed, CF):
    x, wg, experts, shared, dy = _setup(seed)
    k, alpha, beta = 2, 0.3, 0.2
    E = wg.shape[1]
    L0, out0 = _loss(x, wg, experts, shared, k, CF, dy, alpha, beta)
    g = O.layer_backward(x, wg, k, CF, lambda e: experts[e], E, dy, alpha, beta,
                         len(shared), lambda s: shared[s])
    if CF == 0.75:
        assert out0["drop"].sum() > 0            # the case exercises dropped pairs
    eps = 1e-6

    def fd(arr, idx, rebuild):
        old = arr[idx]
        arr[idx] = old + eps
        lp, op = rebuild()
        arr[idx] = old - eps
        lm, om = rebuild()
        arr[idx] = old
        for o in (op, om):                       # the routing must not change
            assert np.array_equal(o["idx"], out0["idx"]) and np.array_equal(o["drop"], out0["drop"])
        return (lp - lm) / (2 * eps)

    rb = lambda: _loss(x, wg, experts, shared, k, CF, dy, alpha, beta)  # noqa: E731
    for idx in np.ndindex(x.shape):
        assert abs(fd(x, idx, rb) - g["dx"][idx]) < 1e-6 * max(1.0, abs(g["dx"][idx]))
    for idx in np.ndindex(wg.shape):
        assert abs(fd(wg, idx, rb) - g["dw_gate"][idx]) < 1e-6 * max(1.0, abs(g["dw_gate"][idx]))
    for e in range(E):
        for m in range(3):
            for idx in list(np.ndindex(experts[e][m].shape))[::3]:
                want = g["dw"][e][m][idx]
                assert abs(fd(experts[e][m], idx, rb) - want) < 1e-6 * max(1.0, abs(want))
    for m in range(3):
        for idx in list(np.ndindex(shared[0][m].shape))[::2]:
            want = g["dw_shared"][0][m][idx]
            assert abs(fd(shared[0][m], idx, rb) - want) < 1e-6 * max(1.0, abs(want))


def test_dense_swiglu_mlp_against_torch_autograd():
    """E = 1, k = 1, no capacity, alpha = beta = 0: the layer is a dense
    SwiGLU MLP (weight 1), whose gradients torch's autograd computes."""
    x, wg, experts, _, dy = _setup(4, T=9, d=6, E=1, k=1, F=7, n_shared=0)
    g = O.layer_backward(x, wg, 1, None, lambda e: experts[e], 1, dy)
    xt = torch.tensor(x, requires_grad=True)
    w1, w3, w2 = (torch.tensor(w, requires_grad=True) for w in experts[0])
    y = (torch.nn.functional.silu(xt @ w1.T) * (xt @ w3.T)) @ w2.T
    (y * torch.tensor(dy)).sum().backward()
    np.testing.assert_allclose(g["dx"], xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    for got, want in zip(g["dw"][0], (w1.grad, w3.grad, w2.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)
    # a single expert always gets weight 1: no gradient reaches the router
    np.testing.assert_allclose(g["dw_gate"], 0.0, atol=1e-12)


@pytest.mark.parametrize("seed,CF", [(3, 0.75), (4, None)])
def test_sampled_backward_equals_full(seed, CF):
    """layer_backward_sampled (unit-by-unit weight gradients, dx at a token
    sample) gives the entries of the finite-difference-pinned layer_backward."""
    x, wg, experts, shared, dy = _setup(seed, T=11, d=6, E=4, k=2, F=5, n_shared=1)
    k, alpha, beta = 2, 0.3, 0.2
    E = wg.shape[1]
    full = O.layer_backward(x, wg, k, CF, lambda e: experts[e], E, dy, alpha, beta,
                            len(shared), lambda s: shared[s])
    tokens = np.array([0, 3, 4, 10])
    units = [(0, 0), (1, 4), (3, 2), (2, 1)]
    sh_units = [(0, 3)]
    smp = O.layer_backward_sampled(x, wg, k, CF, lambda e: experts[e], E, dy, alpha, beta,
                                   tokens, units, len(shared), lambda s: shared[s], sh_units)
    assert np.allclose(smp["dx"], full["dx"][tokens], rtol=1e-12, atol=1e-12)
    assert np.allclose(smp["dw_gate"], full["dw_gate"], rtol=1e-12, atol=1e-12)
    assert np.allclose(smp["dtopk_w"], full["dtopk_w"], rtol=1e-12, atol=1e-12)
    for (e, f), (g1, g3, g2) in smp["dw_units"].items():
        dw1, dw3, dw2 = full["dw"][e]
        assert np.allclose(g1, dw1[f], rtol=1e-12, atol=1e-12)
        assert np.allclose(g3, dw3[f], rtol=1e-12, atol=1e-12)
        assert np.allclose(g2, dw2[:, f], rtol=1e-12, atol=1e-12)
    for (s_, f), (g1, g3, g2) in smp["dws_units"].items():
        dw1, dw3, dw2 = full["dw_shared"][s_]
        assert np.allclose(g1, dw1[f], rtol=1e-12, atol=1e-12)
        assert np.allclose(g3, dw3[f], rtol=1e-12, atol=1e-12)
        assert np.allclose(g2, dw2[:, f], rtol=1e-12, atol=1e-12)
