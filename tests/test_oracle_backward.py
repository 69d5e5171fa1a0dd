"""Pins of the oracle's backward: torch autograd in float64 on the same layer
(rounding off), central finite differences, the degree-one homogeneity
identities of the layer, empty experts, and the rounded mode staying close to
the exact one."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc


def _problem(seed, T=12, H=16, I=8, E=5, k=2):
    rng = np.random.default_rng(seed)
    X = orc.bf16_round(rng.standard_normal((T, H)))
    Wg = orc.bf16_round(rng.standard_normal((E, H, I)) * H ** -0.5)
    Wu = orc.bf16_round(rng.standard_normal((E, H, I)) * H ** -0.5)
    Wd = orc.bf16_round(rng.standard_normal((E, I, H)) * I ** -0.5)
    dY = orc.bf16_round(rng.standard_normal((T, H)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = orc.route(logits, k)
    return X, Wg, Wu, Wd, dY, idx, w


def _torch_layer(X, Wg, Wu, Wd, idx, w):
    """The layer as a per-token sum, differentiable in every input."""
    Y = []
    for t in range(X.shape[0]):
        acc = 0
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            h = torch.nn.functional.silu(X[t] @ Wg[e]) * (X[t] @ Wu[e])
            acc = acc + w[t, j] * (h @ Wd[e])
        Y.append(acc)
    return torch.stack(Y)


def test_backward_matches_torch_autograd_exact_mode():
    X, Wg, Wu, Wd, dY, idx, w = _problem(0)
    tX, tWg, tWu, tWd, tw = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (X, Wg, Wu, Wd, w))
    Y = _torch_layer(tX, tWg, tWu, tWd, idx, tw)
    (Y * torch.from_numpy(dY)).sum().backward()
    g = orc.backward(X, dY, idx, w, Wg, Wu, Wd, exact=True)
    np.testing.assert_allclose(g["dX"], tX.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(g["d_topk_w"], tw.grad.numpy(), rtol=1e-11, atol=1e-13)
    for e in range(Wg.shape[0]):
        np.testing.assert_allclose(g["dW"]["dWg"][e], tWg.grad[e].numpy(), rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(g["dW"]["dWu"][e], tWu.grad[e].numpy(), rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(g["dW"]["dWd"][e], tWd.grad[e].numpy(), rtol=1e-11, atol=1e-13)


def _loss(X, Wg, Wu, Wd, dY, idx, w):
    off, row_token, _, slot_row = orc.dispatch(idx, Wg.shape[0])
    _, O = orc.expert_mlp(X, row_token, off, Wg, Wu, Wd, exact=True)
    return float(np.sum(orc.combine(O, slot_row, w, exact=True) * dY))


def test_backward_finite_differences():
    X, Wg, Wu, Wd, dY, idx, w = _problem(1)
    g = orc.backward(X, dY, idx, w, Wg, Wu, Wd, exact=True)
    eps = 1e-6
    rng = np.random.default_rng(9)
    for name, arr, grad in (("X", X, g["dX"]), ("w", w, g["d_topk_w"])):
        for _ in range(6):
            pos = tuple(rng.integers(0, s) for s in arr.shape)
            p, m = arr.copy(), arr.copy()
            p[pos] += eps
            m[pos] -= eps
            args = {"X": X, "w": w}
            args[name] = p
            lp = _loss(args["X"], Wg, Wu, Wd, dY, idx, args["w"])
            args[name] = m
            lm = _loss(args["X"], Wg, Wu, Wd, dY, idx, args["w"])
            assert abs((lp - lm) / (2 * eps) - grad[pos]) <= 1e-6 * max(1.0, abs(grad[pos]))
    e = int(idx[0, 0])
    for key, W in (("dWg", Wg), ("dWu", Wu), ("dWd", Wd)):
        pos = (e,) + tuple(rng.integers(0, s) for s in W.shape[1:])
        p, m = W.copy(), W.copy()
        p[pos] += eps
        m[pos] -= eps
        ws = {"dWg": (Wg, Wu, Wd), "dWu": (Wg, Wu, Wd), "dWd": (Wg, Wu, Wd)}[key]
        sel = {"dWg": 0, "dWu": 1, "dWd": 2}[key]
        wp, wm = list(ws), list(ws)
        wp[sel], wm[sel] = p, m
        fd = (_loss(X, *wp, dY, idx, w) - _loss(X, *wm, dY, idx, w)) / (2 * eps)
        assert abs(fd - g["dW"][key][e][pos[1:]]) <= 1e-6 * max(1.0, abs(fd))


def test_homogeneity_identities():
    """Y is linear in W_down and in W_up, and linear in w: Euler's theorem gives
    <dW_down, W_down> = <dW_up, W_up> = sum w * dwt = <dY, Y> (rounding off)."""
    X, Wg, Wu, Wd, dY, idx, w = _problem(2, T=30, E=7, k=3)
    g = orc.backward(X, dY, idx, w, Wg, Wu, Wd, exact=True)
    L = _loss(X, Wg, Wu, Wd, dY, idx, w)
    sd = sum(np.sum(g["dW"]["dWd"][e] * Wd[e]) for e in range(7))
    su = sum(np.sum(g["dW"]["dWu"][e] * Wu[e]) for e in range(7))
    sw = np.sum(w * g["d_topk_w"])
    for v in (sd, su, sw):
        assert abs(v - L) <= 1e-10 * max(1.0, abs(L))


def test_empty_experts_get_zero_gradients():
    X, Wg, Wu, Wd, dY, idx, w = _problem(3, T=4, E=20, k=2)
    g = orc.backward(X, dY, idx, w, Wg, Wu, Wd)
    used = set(idx.ravel().tolist())
    for e in range(20):
        if e not in used:
            for key in ("dWg", "dWu", "dWd"):
                assert not np.any(g["dW"][key][e])


def test_rounded_mode_close_to_exact():
    """The bf16 rounding points move the gradients by about one bf16 ulp of the
    summed terms: norm-wise within 1 % of the exact-arithmetic gradients."""
    X, Wg, Wu, Wd, dY, idx, w = _problem(4, T=64, H=64, I=32, E=6, k=2)
    ge = orc.backward(X, dY, idx, w, Wg, Wu, Wd, exact=True)
    gr = orc.backward(X, dY, idx, w, Wg, Wu, Wd)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(gr["dX"], ge["dX"]) < 1e-2
    assert rel(gr["d_topk_w"], ge["d_topk_w"]) < 1e-2
    for key in ("dWg", "dWu", "dWd"):
        for e in range(6):
            assert rel(gr["dW"][key][e], ge["dW"][key][e]) < 1e-2


def test_backward_tokens_matches_full_backward():
    """The per-token path used for sampled checks at full size equals the
    per-expert backward (itself pinned to autograd above), exactly in exact
    mode and after bf16 rounding of dX otherwise."""
    X, Wg, Wu, Wd, dY, idx, w = _problem(4, T=16, E=6, k=3)
    toks = np.array([0, 3, 7, 15])
    for exact in (True, False):
        full = orc.backward(X, dY, idx, w, Wg, Wu, Wd, exact=exact)
        dX, dwt = orc.backward_tokens(X, dY, idx, w, Wg, Wu, Wd, toks, exact=exact)
        np.testing.assert_allclose(dX, full["dX"][toks], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dwt, full["d_topk_w"][toks], rtol=1e-12, atol=1e-14)
