"""GPU parity at the full workload sizes on every element: h and O of every routed row
(expert by expert) and Y of every token, against the oracle, for the four forward workloads
(the prefill shapes with both routings, decode and large MXFP8), in the launch configuration
the benchmark times.  For large MXFP8, rows with an element outside the requantisation
ambiguity get the one of an implementation on the hardware's FP8 block summation
(``check_close_mx``).  The sampled full-size tests (test_gpu_parity_full.py) cover the
training workload's gradients."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc

from gpu_helpers import check_close, check_close_mx, host_weight_fn, mx_block_sum_ambiguity, to_f64
from test_gpu_parity_full import _setup

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("name", ["prefill", "prefill_rankzipf", "decode", "large_mxfp8"])
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
