"""Pins of the oracle's router backward (gradient with respect to the logits):
central finite differences through the forward routing function itself, float64
autograd of the softmax-over-E-renormalised-over-k formulation, and the
invariants (rows sum to zero, unchosen logits get zero, k = E is the plain
softmax backward)."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as orc


def _grid_logits(rng, T, E, step=2.0 ** -8):
    # distinct multiples of 2^-8 in [-4, 4): exact in fp32 with room for exact +-2^-12 steps
    # and no near-ties in the selection
    out = np.empty((T, E), dtype=np.float32)
    for t in range(T):
        out[t] = (rng.choice(2048, E, replace=False) - 1024) * step
    return out


@pytest.mark.parametrize("T,E,k", [(5, 8, 2), (4, 16, 5), (3, 6, 6), (2, 32, 1)])
def test_route_backward_matches_central_differences(T, E, k):
    rng = np.random.default_rng(100 + E + k)
    logits = _grid_logits(rng, T, E)
    dw = rng.standard_normal((T, k))
    g = orc.route_backward(logits, k, dw)
    eps = 2.0 ** -12            # logits +- eps stay exact in fp32 and keep the same top-k set
    for t in range(T):
        for e in range(E):
            lp, lm = logits.copy(), logits.copy()
            lp[t, e] += eps
            lm[t, e] -= eps
            ip, wp = orc.route(lp[t:t + 1], k)
            im, wm = orc.route(lm[t:t + 1], k)
            i0, _ = orc.route(logits[t:t + 1], k)
            assert np.array_equal(ip, i0) and np.array_equal(im, i0)
            fd = ((wp - wm) * dw[t]).sum() / (2 * eps)
            assert abs(fd - g[t, e]) <= 1e-6 * (1 + abs(g[t, e])), (t, e, fd, g[t, e])


@pytest.mark.parametrize("k", [1, 3, 8, 12])
def test_route_backward_matches_autograd_of_full_softmax(k):
    rng = np.random.default_rng(7 + k)
    T, E = 9, 12
    logits = rng.standard_normal((T, E)).astype(np.float32)
    dw = rng.standard_normal((T, k))
    idx, _ = orc.route(logits, k)
    # softmax over all E, gather the chosen, renormalise over them (the other description)
    l = torch.tensor(logits.astype(np.float64), requires_grad=True)
    p = torch.softmax(l, dim=1)
    sel = torch.gather(p, 1, torch.from_numpy(idx.astype(np.int64)))
    w = sel / sel.sum(dim=1, keepdim=True)
    (w * torch.from_numpy(dw)).sum().backward()
    g = orc.route_backward(logits, k, dw)
    assert np.allclose(g, l.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_route_backward_invariants():
    rng = np.random.default_rng(3)
    T, E, k = 50, 64, 6
    logits = rng.standard_normal((T, E)).astype(np.float32)
    dw = rng.standard_normal((T, k)) * 10
    g = orc.route_backward(logits, k, dw)
    idx, w = orc.route(logits, k)
    assert np.allclose(g.sum(axis=1), 0, atol=1e-12)              # shift invariance of the softmax
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    assert np.all(g[~mask] == 0)                                  # unchosen logits
    # a constant gradient on the weights does not move the logits (weights sum to 1)
    assert np.allclose(orc.route_backward(logits, k, np.ones((T, k)) * 3.5), 0, atol=1e-12)
