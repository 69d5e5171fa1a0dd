"""Pins of the oracle's forward (expert MLP + combine): brute force with scalar
loops, reductions to a dense SwiGLU MLP computed with torch, and exact
identities."""
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc


def _rand_bf16(rng, shape, scale=1.0):
    return orc.bf16_round(rng.standard_normal(shape) * scale)


def _torch_dense_swiglu(x, wg, wu, wd):
    """Dense SwiGLU MLP with torch ops, bf16 rounding of h and of the output."""
    x, wg, wu, wd = (torch.from_numpy(a) for a in (x, wg, wu, wd))
    h = torch.nn.functional.silu(x @ wg) * (x @ wu)
    h = h.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    return (h @ wd).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def _layer(X, logits, Wg, Wu, Wd, k, mxfp8=False, exact=False):
    idx, w = orc.route(logits, k)
    off, row_token, row_slot, slot_row = orc.dispatch(idx, Wg.shape[0])
    h, O = orc.expert_mlp(X, row_token, off, Wg, Wu, Wd, mxfp8=mxfp8, exact=exact)
    return orc.combine(O, slot_row, w, exact=exact), (idx, w, off, row_token, slot_row, h, O)


def test_single_expert_is_dense_swiglu_mlp():
    rng = np.random.default_rng(0)
    T, H, I = 33, 64, 32
    X = _rand_bf16(rng, (T, H))
    Wg, Wu = _rand_bf16(rng, (1, H, I), H ** -0.5), _rand_bf16(rng, (1, H, I), H ** -0.5)
    Wd = _rand_bf16(rng, (1, I, H), I ** -0.5)
    Y, _ = _layer(X, rng.standard_normal((T, 1)).astype(np.float32), Wg, Wu, Wd, 1)
    ref = _torch_dense_swiglu(X, Wg[0], Wu[0], Wd[0])
    # torch rounds fp64 -> fp32 -> bf16 (double rounding); allow one bf16 ulp there
    assert np.all(np.abs(Y - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30)
    assert np.mean(Y == ref) > 0.99


def test_all_experts_uniform_identical_is_dense_mlp_bit_exact():
    rng = np.random.default_rng(1)
    T, H, I, E = 20, 64, 32, 8
    X = _rand_bf16(rng, (T, H))
    wg, wu, wd = _rand_bf16(rng, (H, I), 0.125), _rand_bf16(rng, (H, I), 0.125), _rand_bf16(rng, (I, H), 0.2)
    Wg, Wu, Wd = (np.repeat(a[None], E, 0) for a in (wg, wu, wd))
    Y, (idx, w, *_ ) = _layer(X, np.zeros((T, E), np.float32), Wg, Wu, Wd, E)
    assert np.all(w == 1.0 / E)
    _, _, _, O = orc.expert_forward_rows(X, wg, wu, wd)
    assert np.array_equal(Y, O)


def _scalar_layer(X, logits, Wg, Wu, Wd, k):
    """Scalar-loop brute force: route, MLP and combine per token and slot."""
    T, E = logits.shape
    H, I = Wg.shape[1], Wg.shape[2]
    Y = np.zeros((T, H))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        ex = [math.exp(float(logits[t, e]) - float(logits[t, order[0]])) for e in order]
        for j, e in enumerate(order):
            g = [sum(X[t, a] * Wg[e, a, i] for a in range(H)) for i in range(I)]
            u = [sum(X[t, a] * Wu[e, a, i] for a in range(H)) for i in range(I)]
            h = orc.bf16_round(np.array([g[i] / (1 + math.exp(-g[i])) * u[i] for i in range(I)]))
            o = orc.bf16_round(np.array([sum(h[i] * Wd[e, i, c] for i in range(I)) for c in range(H)]))
            Y[t] += ex[j] / sum(ex) * o
    return orc.bf16_round(Y)


def test_brute_force_scalar_loops():
    rng = np.random.default_rng(2)
    T, H, I, E, k = 6, 8, 4, 5, 2
    X = _rand_bf16(rng, (T, H))
    Wg, Wu = _rand_bf16(rng, (E, H, I), 0.35), _rand_bf16(rng, (E, H, I), 0.35)
    Wd = _rand_bf16(rng, (E, I, H), 0.5)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    Y, _ = _layer(X, logits, Wg, Wu, Wd, k)
    ref = _scalar_layer(X, logits, Wg, Wu, Wd, k)
    assert np.all(np.abs(Y - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-12)


def test_per_token_definition_matches_dispatched_pipeline():
    rng = np.random.default_rng(3)
    T, H, I, E, k = 40, 64, 32, 8, 3
    X = _rand_bf16(rng, (T, H))
    Wg, Wu = _rand_bf16(rng, (E, H, I), 0.125), _rand_bf16(rng, (E, H, I), 0.125)
    Wd = _rand_bf16(rng, (E, I, H), 0.18)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    Y, (idx, w, *_ ) = _layer(X, logits, Wg, Wu, Wd, k)
    toks = [0, 5, 39, 17]
    Yt = orc.layer_forward_tokens(X, idx, w, Wg, Wu, Wd, toks)
    assert np.array_equal(Yt, Y[toks])


def test_exact_identities():
    rng = np.random.default_rng(4)
    T, H, I, E = 24, 64, 32, 6
    X = _rand_bf16(rng, (T, H))
    Wg, Wu = _rand_bf16(rng, (E, H, I), 0.125), _rand_bf16(rng, (E, H, I), 0.125)
    Wd = _rand_bf16(rng, (E, I, H), 0.18)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    # W_down * 2 (exact in bf16) doubles every output exactly
    Y1, _ = _layer(X, logits, Wg, Wu, Wd, 2)
    Y2, _ = _layer(X, logits, Wg, Wu, 2 * Wd, 2)
    assert np.array_equal(Y2, 2 * Y1)
    # k = 1: the weight is exactly 1 and Y is a permutation of the expert rows
    Y, (idx, w, off, row_token, slot_row, h, O) = _layer(X, logits, Wg, Wu, Wd, 1)
    assert np.all(w == 1.0) and np.array_equal(Y, O[slot_row])
    # a zero weight contributes exactly nothing
    idx, w = orc.route(logits, 2)
    w0 = w.copy()
    w0[:, 1] = 0.0
    off, row_token, _, slot_row = orc.dispatch(idx, E)
    _, O = orc.expert_mlp(X, row_token, off, Wg, Wu, Wd)
    assert np.array_equal(orc.combine(O, slot_row, w0), orc.bf16_round(w0[:, :1] * O[slot_row.reshape(-1, 2)[:, 0]]))


def test_empty_experts_and_subset():
    rng = np.random.default_rng(5)
    T, H, I, E = 10, 64, 32, 50
    X = _rand_bf16(rng, (T, H))
    Wg, Wu = _rand_bf16(rng, (E, H, I), 0.125), _rand_bf16(rng, (E, H, I), 0.125)
    Wd = _rand_bf16(rng, (E, I, H), 0.18)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = orc.route(logits, 2)
    off, row_token, _, slot_row = orc.dispatch(idx, E)
    active = np.nonzero(np.diff(off))[0]
    assert len(active) < E
    Wg2 = Wg.copy()
    Wg2[np.setdiff1d(np.arange(E), active)] = np.nan      # never read
    h1, O1 = orc.expert_mlp(X, row_token, off, Wg, Wu, Wd)
    h2, O2 = orc.expert_mlp(X, row_token, off, Wg2, Wu, Wd)
    assert np.array_equal(O1, O2) and np.isfinite(O2).all()


def test_mxfp8_equals_bf16_on_representable_inputs():
    """With every GEMM operand exactly representable in MXFP8 the fp8 layer
    equals the bf16 layer; with random inputs it stays close."""
    rng = np.random.default_rng(6)
    T, H, I, E, k = 16, 64, 32, 4, 2
    X = orc.mx_fake_quant(_rand_bf16(rng, (T, H)))
    Wg = np.stack([orc.mx_fake_quant(_rand_bf16(rng, (I, H), 0.125)).T for _ in range(E)])
    Wu = np.stack([orc.mx_fake_quant(_rand_bf16(rng, (I, H), 0.125)).T for _ in range(E)])
    Wd = np.stack([orc.mx_fake_quant(_rand_bf16(rng, (H, I), 0.18)).T for _ in range(E)])
    logits = rng.standard_normal((T, E)).astype(np.float32)
    _, (idx, w, off, row_token, slot_row, h, O) = _layer(X, logits, Wg, Wu, Wd, k)
    hq = orc.mx_fake_quant(h)
    # the down projection in the fp8 layer uses the quantised h
    _, (_, _, _, _, _, h8, O8) = _layer(X, logits, Wg, Wu, Wd, k, mxfp8=True)
    assert np.array_equal(h8, h)
    ref = np.concatenate([orc.bf16_round(hq[off[e]:off[e + 1]] @ Wd[e]) for e in range(E)])
    assert np.array_equal(O8, ref)
    Y8, _ = _layer(_rand_bf16(rng, (T, H)), logits, Wg, Wu, Wd, k, mxfp8=True)
    assert np.isfinite(Y8).all()
