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


# ------------------------------------------------------------------------------------------
# Rounded-mode pin: the backward of the rounded layer (h rounded to bf16 as in the forward;
# dO = w dY, P, dg, du exact; dX and dW rounded once after exact sums) written as plain scalar
# loops over tokens, slots and elements, with a bf16 rounding of its own (Python's round() is
# round-half-even on the exactly scaled significand).  Nothing here calls the oracle's code.
# ------------------------------------------------------------------------------------------
import math


def _rnd_bf16(x: float) -> float:
    if x == 0.0:
        return x
    m, e = math.frexp(x)                     # x = m 2^e, 0.5 <= |m| < 1: 8 significant bits
    return math.ldexp(round(math.ldexp(m, 8)), e - 8)


def _near_bf16_midpoint(x: float, eps: float = 1e-6) -> bool:
    """Whether x lies within eps bf16 steps of a rounding midpoint (either rounding is then a
    matter of the summation order)."""
    if x == 0.0:
        return False
    m, e = math.frexp(x)
    f = abs(math.ldexp(m, 8))
    return abs(f - math.floor(f) - 0.5) < eps


def _scalar_backward(X, dY, idx, w, Wg, Wu, Wd, round_h=True, round_dO=False):
    T, H = len(X), len(X[0])
    k = len(idx[0])
    E, I = len(Wg), len(Wg[0][0])
    sig = lambda v: 1.0 / (1.0 + math.exp(-v))
    dX = [[0.0] * H for _ in range(T)]
    dwt = [[0.0] * k for _ in range(T)]
    dWg = [[[0.0] * I for _ in range(H)] for _ in range(E)]
    dWu = [[[0.0] * I for _ in range(H)] for _ in range(E)]
    dWd = [[[0.0] * H for _ in range(I)] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            e, wt = int(idx[t][j]), float(w[t][j])
            for i in range(I):
                g = sum(X[t][c] * Wg[e][c][i] for c in range(H))
                u = sum(X[t][c] * Wu[e][c][i] for c in range(H))
                s = sig(g)
                h = g * s * u
                if round_h:
                    h = _rnd_bf16(h)
                p = sum(dY[t][c] * Wd[e][i][c] for c in range(H))
                dwt[t][j] += h * p
                dh = wt * p
                du = dh * g * s                          # d(h)/du = silu(g)
                dg = dh * u * s * (1.0 + g * (1.0 - s))  # d(h)/dg = u silu'(g)
                for c in range(H):
                    dX[t][c] += dg * Wg[e][c][i] + du * Wu[e][c][i]
                    dWg[e][c][i] += X[t][c] * dg
                    dWu[e][c][i] += X[t][c] * du
                    dO = wt * dY[t][c]
                    if round_dO:
                        dO = _rnd_bf16(dO)
                    dWd[e][i][c] += h * dO
    return dX, dwt, dWg, dWu, dWd


def _mismatches(unrounded, got, path=()):
    """Elements where bf16(unrounded) differs from got, other than at rounding midpoints."""
    if isinstance(unrounded, list):
        out = []
        for n, (a, b) in enumerate(zip(unrounded, got)):
            out += _mismatches(a, b, path + (n,))
        return out
    if _rnd_bf16(unrounded) != float(got) and not _near_bf16_midpoint(unrounded):
        return [path]
    return []


def _pin_problem():
    X, Wg, Wu, Wd, dY, idx, w = _problem(11, T=6, H=8, I=4, E=3, k=2)
    return X, Wg, Wu, Wd, dY, idx, w


def test_rounded_backward_matches_scalar_loops():
    """The oracle's rounded backward equals the scalar-loop definition element by element: dX,
    dW_gate, dW_up and dW_down bit for bit after one bf16 rounding (up to ties the summation
    order decides), d_topk_w to float64 rounding."""
    X, Wg, Wu, Wd, dY, idx, w = _pin_problem()
    assert len(set(idx.ravel().tolist())) == 3            # every expert has rows
    g = orc.backward(X, dY, idx, w, Wg, Wu, Wd)
    dX, dwt, dWg, dWu, dWd = _scalar_backward(X.tolist(), dY.tolist(), idx.tolist(), w.tolist(),
                                              Wg.tolist(), Wu.tolist(), Wd.tolist())
    assert _mismatches(dX, g["dX"].tolist()) == []
    for name, ref in (("dWg", dWg), ("dWu", dWu), ("dWd", dWd)):
        got = [g["dW"][name][e].tolist() for e in range(3)]
        assert _mismatches(ref, got) == [], name
    np.testing.assert_allclose(g["d_topk_w"], np.array(dwt), rtol=1e-12, atol=1e-14)


def test_scalar_pin_tells_rounding_points_apart():
    """The scalar-loop comparison above would catch a rounding point in the wrong place: an
    oracle that rounded dO = w dY to bf16, or that did not round h, disagrees with the
    definition on some dW_down elements of the same problem."""
    X, Wg, Wu, Wd, dY, idx, w = _pin_problem()
    g = orc.backward(X, dY, idx, w, Wg, Wu, Wd)
    got = [g["dW"]["dWd"][e].tolist() for e in range(3)]
    args = (X.tolist(), dY.tolist(), idx.tolist(), w.tolist(), Wg.tolist(), Wu.tolist(), Wd.tolist())
    assert _mismatches(_scalar_backward(*args, round_dO=True)[4], got) != []
    assert _mismatches(_scalar_backward(*args, round_h=False)[4], got) != []
