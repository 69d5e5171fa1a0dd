"""Pins of the oracle's activations h = f(G, U) (and the ungated ReLU^2, h = f(U))
and their derivatives: textbook values (sigmoid(1), the normal CDF at 1, squares),
GELU's odd-part identity, the clamps' limit cases, and the derivatives against
float64 autograd of the forward functions and against central differences."""
import math

import numpy as np
import pytest
import torch

import oracle.moe_oracle as orc

LIMIT = {"swiglu_clamp": 10.0, "swiglu_oai": 7.0}


def _gu(rng, n=400, scale=4.0):
    G = rng.uniform(-scale, scale, n)
    U = rng.uniform(-scale, scale, n)
    return G, U


def test_textbook_values():
    sig1 = 0.7310585786300049          # 1 / (1 + e^-1)
    phi1 = 0.8413447460685429          # standard normal CDF at 1
    assert orc.activation(1.0, 2.0, "swiglu") == pytest.approx(2 * sig1, rel=1e-15)
    assert orc.activation(1.0, 3.0, "geglu") == pytest.approx(3 * phi1, rel=1e-15)
    assert orc.activation(-1.5, 3.0, "reglu") == 0.0
    assert orc.activation(1.5, 3.0, "reglu") == 4.5
    # SwiGLU-OAI: g sigmoid(1.702 g) (u + 1)
    assert orc.activation(2.0, 0.0, "swiglu_oai", 7.0) == pytest.approx(2.0 / (1.0 + math.exp(-3.404)), rel=1e-15)
    assert orc.activation(2.0, -1.0, "swiglu_oai", 7.0) == 0.0
    # ReLU^2: max(U, 0)^2, no gate
    assert orc.activation(None, 3.0, "relu2") == 9.0
    assert orc.activation(-5.0, 1.5, "relu2") == 2.25
    assert orc.activation(5.0, -2.0, "relu2") == 0.0
    assert orc.activation_grads(None, np.array([3.0, -2.0, 0.0]), "relu2")[1].tolist() == [6.0, 0.0, 0.0]
    assert orc.activation_grads(None, 3.0, "relu2")[0] is None


def test_gelu_odd_part_and_limits():
    x = np.linspace(-6, 6, 97)
    g = orc.activation(x, 1.0, "geglu")
    gm = orc.activation(-x, 1.0, "geglu")
    assert np.allclose(g - gm, x, atol=1e-14)                 # Phi(x) + Phi(-x) = 1
    assert abs(orc.activation(30.0, 1.0, "geglu") - 30.0) < 1e-12
    assert abs(orc.activation(-30.0, 1.0, "geglu")) < 1e-12


def test_clamps():
    rng = np.random.default_rng(1)
    G, U = _gu(rng, scale=5.0)
    # inside the bounds the bounded SwiGLU is the plain SwiGLU
    assert np.array_equal(orc.activation(G, U, "swiglu_clamp", 10.0), orc.activation(G, U, "swiglu"))
    # outside: the gate is capped from above only, the up value on both sides
    assert orc.activation(12.0, 3.0, "swiglu_clamp", 10.0) == orc.activation(10.0, 3.0, "swiglu")
    assert orc.activation(-12.0, 3.0, "swiglu_clamp", 10.0) == orc.activation(-12.0, 3.0, "swiglu")
    assert orc.activation(1.0, 13.0, "swiglu_clamp", 10.0) == orc.activation(1.0, 10.0, "swiglu")
    assert orc.activation(1.0, -13.0, "swiglu_clamp", 10.0) == orc.activation(1.0, -10.0, "swiglu")
    assert orc.activation(9.0, 8.0, "swiglu_oai", 7.0) == orc.activation(7.0, 7.0, "swiglu_oai", 7.0)
    with pytest.raises(ValueError):
        orc.activation(G, U, "swiglu_clamp", None)


def _torch_forward(g, u, act, lim):
    if act == "swiglu":
        return torch.nn.functional.silu(g) * u
    if act == "swiglu_clamp":
        gc = torch.clamp(g, max=lim)
        return torch.nn.functional.silu(gc) * torch.clamp(u, -lim, lim)
    if act == "swiglu_oai":
        gc = torch.clamp(g, max=lim)
        return gc * torch.sigmoid(1.702 * gc) * (torch.clamp(u, -lim, lim) + 1)
    if act == "geglu":
        return torch.nn.functional.gelu(g) * u
    if act == "relu2":
        return torch.relu(u) ** 2
    return torch.relu(g) * u


@pytest.mark.parametrize("act", orc.ACTIVATIONS)
def test_grads_match_autograd(act):
    rng = np.random.default_rng(11 + orc.ACTIVATIONS.index(act))
    G, U = _gu(rng, scale=12.0)
    G = G[np.abs(np.abs(G) - LIMIT.get(act, 1e9)) > 1e-3]    # away from the clamp kinks
    U = U[: G.size]
    lim = LIMIT.get(act)
    g = torch.tensor(G, requires_grad=True)
    u = torch.tensor(U, requires_grad=True)
    _torch_forward(g, u, act, lim).sum().backward()
    fg, fu = orc.activation_grads(G, U, act, lim)
    if orc.is_gated(act):
        assert np.allclose(fg, g.grad.numpy(), rtol=1e-12, atol=1e-13)
    else:
        assert fg is None and g.grad is None
    assert np.allclose(fu, u.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(orc.activation(G, U, act, lim), _torch_forward(g, u, act, lim).detach().numpy(),
                       rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("act", orc.ACTIVATIONS)
def test_grads_match_central_differences(act):
    rng = np.random.default_rng(7)
    G, U = _gu(rng, n=200, scale=9.0)
    lim = LIMIT.get(act)
    keep = np.abs(G) > 1e-3                                       # away from the ReGLU kink
    if lim:
        keep &= (np.abs(np.abs(G) - lim) > 1e-3) & (np.abs(np.abs(U) - lim) > 1e-3)
    G, U = G[keep], U[keep]
    eps = 1e-6
    fg, fu = orc.activation_grads(G, U, act, lim)
    dg = (orc.activation(G + eps, U, act, lim) - orc.activation(G - eps, U, act, lim)) / (2 * eps)
    du = (orc.activation(G, U + eps, act, lim) - orc.activation(G, U - eps, act, lim)) / (2 * eps)
    if orc.is_gated(act):
        assert np.allclose(fg, dg, rtol=1e-6, atol=1e-7)
    else:
        assert fg is None and np.all(dg == 0)
    assert np.allclose(fu, du, rtol=1e-6, atol=1e-7)


def test_layer_backward_with_activation_matches_autograd():
    # the whole backward of one expert under a non-default activation, exact mode
    rng = np.random.default_rng(5)
    n, H, I = 6, 16, 8
    x = rng.standard_normal((n, H))
    dy = rng.standard_normal((n, H))
    w = rng.uniform(0.1, 1.0, n)
    wg, wu, wd = (rng.standard_normal(s) / 3 for s in ((H, I), (H, I), (I, H)))
    for act in orc.ACTIVATIONS:
        lim = LIMIT.get(act)
        gated = orc.is_gated(act)
        r = orc.expert_backward_rows(x, dy, w, wg if gated else None, wu, wd, exact=True, act=act, limit=lim)
        tx, twg, twu, twd = (torch.tensor(a, requires_grad=True) for a in (x, wg, wu, wd))
        h = _torch_forward(tx @ twg, tx @ twu, act, lim)
        o = h @ twd
        (torch.tensor(w)[:, None] * o * torch.tensor(dy)).sum().backward()
        if gated:
            assert np.allclose(r["dWg"], twg.grad.numpy(), rtol=1e-10, atol=1e-12), act
        else:
            assert r["dWg"] is None and r["dg"] is None
        assert np.allclose(r["dWu"], twu.grad.numpy(), rtol=1e-10, atol=1e-12), act
        assert np.allclose(r["dXr"], tx.grad.numpy(), rtol=1e-10, atol=1e-12), act
        assert np.allclose(r["dWd"], twd.grad.numpy(), rtol=1e-10, atol=1e-12), act
