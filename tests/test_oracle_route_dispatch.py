"""Pins of the oracle's routing and dispatch: brute force on tiny inputs,
closed forms, a library softmax special case and the dispatch invariants
(each token appears exactly k times, per-expert counts sum to T*k, the
inverse map is a bijection, rows ascend by token inside an expert)."""
import math

import numpy as np
import pytest
import scipy.special

from oracle import moe_oracle as orc
from grouped_gemm_router_amd import workloads as wl


def _brute_route(logits, k):
    T, E = logits.shape
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        idx[t] = order
        den = sum(math.exp(float(logits[t, e]) - float(logits[t, order[0]])) for e in order)
        w[t] = [math.exp(float(logits[t, e]) - float(logits[t, order[0]])) / den for e in order]
    return idx, w


@pytest.mark.parametrize("T,E,k", [(7, 5, 1), (9, 8, 3), (16, 16, 16), (5, 33, 4)])
def test_route_brute_force(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, :] = np.float32(0.5)                    # a row of ties
    logits[1, ::2] = logits[1, 1]                     # partial ties
    idx, w = orc.route(logits, k)
    bi, bw = _brute_route(logits, k)
    assert np.array_equal(idx, bi)
    np.testing.assert_allclose(w, bw, rtol=1e-14, atol=0)


def test_route_k_equals_e_is_softmax():
    rng = np.random.default_rng(3)
    logits = (rng.standard_normal((50, 12)) * 3).astype(np.float32)
    idx, w = orc.route(logits, 12)
    ref = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(ref, idx.astype(np.int64), 1), rtol=1e-13)


def test_route_top2_closed_form_and_invariants():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((200, 9)).astype(np.float32)
    idx, w = orc.route(logits, 2)
    l0 = np.take_along_axis(logits, idx[:, :1].astype(np.int64), 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(logits, idx[:, 1:].astype(np.int64), 1)[:, 0].astype(np.float64)
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-14)
    for k in (1, 3, 9):
        idx, w = orc.route(logits, k)
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=k * 2.0 ** -52)
        assert np.all(np.diff(w, axis=1) <= 0) and np.all(w[:, 0] >= 1.0 / k)
        assert all(len(set(r)) == k for r in idx.tolist())


def test_route_uniform_and_signed_zero_ties():
    logits = np.zeros((4, 8), np.float32)
    logits[1, :] = -0.0
    logits[2, 3] = -0.0
    logits[3, :4] = -0.0
    idx, w = orc.route(logits, 4)
    assert np.array_equal(idx, np.tile(np.arange(4, dtype=np.int32), (4, 1)))
    assert np.all(w == 0.25)


def _brute_dispatch(idx, E):
    T, k = idx.shape
    offsets, row_token, row_slot = [0], [], []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    row_token.append(t)
                    row_slot.append(t * k + j)
        offsets.append(len(row_token))
    slot_row = [0] * (T * k)
    for r, s in enumerate(row_slot):
        slot_row[s] = r
    return [np.array(a, np.int32) for a in (offsets, row_token, row_slot, slot_row)]


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (13, 8, 2), (40, 64, 8), (3, 300, 3)])
def test_dispatch_brute_force(T, E, k):
    rng = np.random.default_rng(T + E + k)
    idx, _ = orc.route(rng.standard_normal((T, E)).astype(np.float32), k)
    got = orc.dispatch(idx, E)
    for g, b in zip(got, _brute_dispatch(idx, E)):
        assert g.dtype == np.int32 and np.array_equal(g, b)


@pytest.mark.parametrize("name", ["tiny", "prefill", "decode", "large_mxfp8", "train"])
def test_dispatch_invariants_on_workloads(name):
    cfg = wl.config(name)
    idx, w = orc.route(wl.make_logits(cfg), cfg.k)
    offsets, row_token, row_slot, slot_row = orc.dispatch(idx, cfg.E)
    A = cfg.T * cfg.k
    counts = np.diff(offsets)
    assert offsets[0] == 0 and offsets[-1] == A and np.all(counts >= 0)
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=cfg.E))
    assert np.array_equal(np.bincount(row_token, minlength=cfg.T), np.full(cfg.T, cfg.k))
    assert np.array_equal(np.sort(row_slot), np.arange(A)) and np.array_equal(row_slot[slot_row], np.arange(A))
    assert np.array_equal(row_token, row_slot // cfg.k)
    for e in np.nonzero(counts)[0]:
        seg = row_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(idx.ravel()[row_slot[offsets[e]:offsets[e + 1]]] == e)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-12)


def test_workload_routing_structure():
    """The skewed bias sends every prefill token to the same 8 experts."""
    cfg = wl.config("prefill")
    idx, _ = orc.route(wl.make_logits(cfg), cfg.k)
    assert len(np.unique(idx)) == 8
    cfg = wl.config("decode")
    idx, _ = orc.route(wl.make_logits(cfg), cfg.k)
    assert 120 < len(np.unique(idx)) < 200
