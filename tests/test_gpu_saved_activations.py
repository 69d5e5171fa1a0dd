"""GPU parity of the training pair that keeps the projections (moe_expert_mlp_save +
moe_backward_saved) against the CPU oracle: the saved G and U of every routed row, the
forward's h, O and Y, and every gradient, on the small and ragged problems of the recompute
path's tests (every row class, every activation).  The saved G and U are the same fp32
accumulations the recompute forms (same k order per output element), and the elementwise pass
forms dg, du and w h from them and from P with the recompute's expressions, so dX and the weight
gradients must also equal the recompute path's bit for bit."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc
from grouped_gemm_router_amd import workloads as wl

from gpu_helpers import (H_RESCUE, backward_h_ambiguity, check_close, device_weights, host_weight_fn, to_bits,
                         to_dev, to_f64)
from test_gpu_parity_small import ACTS, BWD, REMAINDER_COUNTS, remainder_logits

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _run(cfg, logits, act="swiglu", limit=0.0):
    from grouped_gemm_router_amd.layer import MoELayer
    gated = orc.is_gated(act)
    X, dY = wl.make_x(cfg), wl.make_dy(cfg)
    W = {n: device_weights(cfg, n) for n in (("gate", "up", "down") if gated else ("up", "down"))}
    out = {}
    for saved in (True, False):
        layer = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, activation=act, act_limit=limit,
                         save_activations=saved).load_weights(W.get("gate"), W["up"], W["down"])
        Y = layer.forward(torch.from_numpy(logits).cuda(), to_dev(X), backward_plan=True)
        grads = layer.backward(to_dev(X), to_dev(dY))
        torch.cuda.synchronize()
        pl = layer.plan(cfg.T, True)
        out[saved] = {"Y": Y.clone(), "grads": [g.clone() if g is not None else None for g in grads],
                      "pl": pl, "layer": layer}
    return X, dY, out


def _check(cfg, logits, act, limit, X, dY, out):
    gated = orc.is_gated(act)
    lim = limit or None
    fn = lambda n: host_weight_fn(cfg, n)
    idx, w = orc.route(logits, cfg.k)
    off, row_token, row_slot, slot_row = orc.dispatch(idx, cfg.E)
    s = out[True]
    pl = s["pl"]
    assert np.array_equal(pl["offsets"].cpu().numpy(), off)
    # the saved projections, h and O of every row, and Y
    GU = pl["GU"].cpu().numpy().astype(np.float64)
    Xv = orc.bf16_decode(X)
    h_all = np.zeros((cfg.T * cfg.k, cfg.I))
    O_all = np.zeros((cfg.T * cfg.k, cfg.H))
    for e in range(cfg.E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        wg = orc.bf16_decode(fn("gate")(e)) if gated else None
        wu, wd = (orc.bf16_decode(fn(n)(e)) for n in ("up", "down"))
        G, U, h, O = orc.expert_forward_rows(Xv[row_token[lo:hi]], wg, wu, wd, act=act, limit=lim)
        if gated:
            check_close(GU[lo:hi, :cfg.I], G, f"{act} saved G[{e}]")
        check_close(GU[lo:hi, cfg.I:], U, f"{act} saved U[{e}]")
        h_all[lo:hi], O_all[lo:hi] = h, O
    n = off[-1]
    check_close(to_f64(pl["H_rows"])[:n], h_all[:n], f"{act} h")
    check_close(to_f64(pl["O_rows"])[:n], O_all[:n], f"{act} O")
    check_close(to_f64(s["Y"]), orc.combine(O_all, slot_row, w), f"{act} Y")
    # gradients against the oracle
    dX, dWg, dWu, dWd, dtw = s["grads"]
    ref = orc.backward(X, dY, idx, w, fn("gate") if gated else None, fn("up"), fn("down"), E=cfg.E, act=act,
                       limit=lim)
    amb_dwd, amb_dtw = backward_h_ambiguity(cfg, X, dY, idx, w, fn, act, lim)
    check_close(to_f64(dX), ref["dX"], f"{act} dX")
    check_close(dtw.cpu().numpy(), ref["d_topk_w"], f"{act} d_topk_w", ambiguity=amb_dtw, max_rescued=H_RESCUE)
    if not gated:
        assert dWg is None
    for key, t in (("dWg", dWg), ("dWu", dWu), ("dWd", dWd)):
        if t is None:
            continue
        g = to_f64(t)
        for e in range(cfg.E):
            check_close(g[e], ref["dW"][key][e], f"{act} {key}[{e}]",
                        ambiguity=amb_dwd.get(e) if key == "dWd" else None, max_rescued=H_RESCUE)
    # the recompute path's dX and weight gradients, bit for bit
    for name, a, b in zip(("dX", "dWg", "dWu", "dWd"), s["grads"][:4], out[False]["grads"][:4]):
        if a is None:
            assert b is None
            continue
        assert np.array_equal(to_bits(a), to_bits(b)), f"{act} {name}: saved and recompute paths differ"


@pytest.mark.parametrize("cfg", BWD, ids=[c.name for c in BWD])
def test_saved_backward_small_vs_oracle(cfg):
    _say("saved backward", cfg)
    logits = wl.make_logits(cfg)
    X, dY, out = _run(cfg, logits)
    _check(cfg, logits, "swiglu", 0.0, X, dY, out)
    # a second backward from the same saved projections gives the same bits
    s = out[True]
    first = [to_bits(t).copy() for t in s["grads"][:4]] + [s["grads"][4].cpu().numpy().copy()]
    again = s["layer"].backward(to_dev(X), to_dev(dY))
    torch.cuda.synchronize()
    for a, b in zip(first, [to_bits(t) for t in again[:4]] + [again[4].cpu().numpy()]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("act", ["swiglu", "relu2"])
def test_saved_every_row_class(act):
    _say("saved row classes", act, REMAINDER_COUNTS)
    E = len(REMAINDER_COUNTS)
    logits = remainder_logits(REMAINDER_COUNTS, E, 61)
    cfg = wl.config("tiny", name="row_classes", T=logits.shape[0], H=192, I=128, E=E, k=1, seed=61, backward=True)
    X, dY, out = _run(cfg, logits, act)
    _check(cfg, logits, act, 0.0, X, dY, out)


@pytest.mark.parametrize("act,limit", ACTS, ids=[f"{a}{l:g}" for a, l in ACTS])
def test_saved_activations_vs_oracle(act, limit):
    cfg = wl.config("tiny", name="act_bwd", T=300, H=320, I=192, E=5, k=3, seed=54, backward=True)
    _say("saved", act, limit, cfg)
    logits = wl.make_logits(cfg)
    X, dY, out = _run(cfg, logits, act, limit)
    _check(cfg, logits, act, limit, X, dY, out)

