"""GPU parity at the full workload sizes on every element: h and O of every routed row
(expert by expert) and Y of every token, against the oracle, for the five forward workloads
(the prefill shapes with both routings, decode, large MXFP8 and the training forward, whose
experts of 447-572 rows run every remainder-tile class), in the launch configuration
the benchmark times.  For large MXFP8, rows with an element outside the requantisation
ambiguity get the one of an implementation on the hardware's FP8 block summation
(``check_close_mx``).  The training workload's backward is checked the same way, every
element of every gradient, on both training paths."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc

from gpu_helpers import check_close, check_close_mx, host_weight_fn, mx_block_sum_ambiguity, to_f64
from test_gpu_parity_full import _setup

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("name", ["prefill", "prefill_rankzipf", "decode", "large_mxfp8", "train"])
def test_forward_every_element(name):
    cfg, layer, logits, X, idx, w = _setup(name)
    pl = layer.plan(cfg.T)
    off, row_token, row_slot, slot_row = orc.dispatch(idx, cfg.E)
    assert np.array_equal(pl["offsets"].cpu().numpy(), off)
    fn = lambda n: host_weight_fn(cfg, n)
    mx = cfg.dtype == "mxfp8"
    Xv = orc.bf16_decode(X)
    A = int(off[-1])
    O_ref = np.empty((A, cfg.H))
    amb_O = np.zeros((A, cfg.H)) if mx else None
    active = [e for e in range(cfg.E) if off[e + 1] > off[e]]
    _say(name, "checking every row of", len(active), "experts")
    for e in active:
        lo, hi = int(off[e]), int(off[e + 1])
        wg, wu, wd = (orc.bf16_decode(fn(n)(e)) for n in ("gate", "up", "down"))
        xr = Xv[row_token[lo:hi]]
        G, U, h, O = orc.expert_forward_rows(xr, wg, wu, wd, mxfp8=mx)
        check_close(to_f64(pl["H_rows"][lo:hi]), h, f"{name} h[expert {e}]")
        if mx:
            amb_O[lo:hi] = check_close_mx(to_f64(pl["O_rows"][lo:hi]), O, f"{name} O[expert {e}]",
                                          orc.mx_down_ambiguity(G, U, wd),
                                          lambda rows: mx_block_sum_ambiguity(xr[rows], wg, wu, wd))
        else:
            check_close(to_f64(pl["O_rows"][lo:hi]), O, f"{name} O[expert {e}]")
        O_ref[lo:hi] = O
    Y_ref = orc.combine(O_ref, slot_row, w)
    amb_Y = None
    if mx:   # what the valid alternative requantisations of h can change in each token's sum
        amb_Y = np.zeros((cfg.T, cfg.H))
        for j in range(cfg.k):
            r = slot_row[j::cfg.k]
            amb_Y += np.where(r[:, None] >= 0, w[:, j:j + 1] * amb_O[np.maximum(r, 0)], 0.0)
    check_close(to_f64(pl["Y"]), Y_ref, f"{name} Y[every token]", ambiguity=amb_Y)


def test_backward_every_element():
    """The training workload's backward on every element: dX of every token, d_topk_w of every
    slot and the three weight gradients of every expert against the oracle, and the pair that
    keeps the projections (moe_expert_mlp_save + moe_backward_saved) equal to the recompute path
    on dX and every weight gradient, bit for bit."""
    from gpu_helpers import H_RESCUE, backward_h_ambiguity, to_bits, to_dev
    from grouped_gemm_router_amd import workloads as wl
    cfg, layer, logits, X, idx, w = _setup("train", backward=True)
    _, layer_s, _, _, _, _ = _setup("train", backward=True, saved=True)
    dY = wl.make_dy(cfg)
    g = [t.clone() if t is not None else None for t in layer.backward(to_dev(X), to_dev(dY))]
    gs = layer_s.backward(to_dev(X), to_dev(dY))
    torch.cuda.synchronize()
    for name, a, b in zip(("dX", "dW_gate", "dW_up", "dW_down"), g[:4], gs[:4]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name}: saved and recompute paths differ"
    dtw_s = gs[4].cpu().numpy()
    del layer_s, gs
    _say("train backward done on GPU; oracle over every expert")
    fn = lambda n: host_weight_fn(cfg, n)
    ref = orc.backward(X, dY, idx, w, fn("gate"), fn("up"), fn("down"), E=cfg.E)
    amb_dwd, amb_dtw = backward_h_ambiguity(cfg, X, dY, idx, w, fn)
    dX, dWg, dWu, dWd, dtw = g
    check_close(to_f64(dX), ref["dX"], "dX[every token]")
    check_close(dtw.cpu().numpy(), ref["d_topk_w"], "d_topk_w[every slot]", ambiguity=amb_dtw, max_rescued=H_RESCUE)
    check_close(dtw_s, ref["d_topk_w"], "saved-path d_topk_w[every slot]", ambiguity=amb_dtw, max_rescued=H_RESCUE)
    for key, t in (("dWg", dWg), ("dWu", dWu), ("dWd", dWd)):
        for e in range(cfg.E):
            check_close(to_f64(t[e]), ref["dW"][key][e], f"{key}[{e}]",
                        ambiguity=amb_dwd.get(e) if key == "dWd" else None, max_rescued=H_RESCUE)
