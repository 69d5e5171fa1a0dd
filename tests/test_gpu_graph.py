"""HIP-graph capture of the layer: a captured forward (and forward + backward)
replayed several times, with eager work on other inputs through the same plan
buffers between the replays, gives the eager result bit for bit every time, and
that result matches the oracle (routing bit for bit, outputs and gradients within
the layer tolerance), on the recompute and the saved-projection training paths.
No call of the library allocates or clears memory with a memset, so the whole
step can be captured."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc
from grouped_gemm_router_amd import workloads as wl

from gpu_helpers import (H_RESCUE, backward_h_ambiguity, check_close, device_weights, host_weight_fn,
                         oracle_forward, to_bits, to_dev)

pytestmark = pytest.mark.gpu

CASES = [
    wl.config("tiny", name="graph_rows", T=300, H=320, I=192, E=5, k=3, seed=41, backward=True),
    wl.config("tiny", name="graph_decode", T=24, H=256, I=128, E=64, k=4, seed=42),
    wl.config("tiny", name="graph_mx", T=96, H=256, I=128, E=6, k=2, dtype="mxfp8", seed=43),
    wl.config("tiny", name="graph_relu2", T=300, H=320, I=192, E=5, k=3, seed=44, backward=True, activation="relu2"),
    # the training pair that keeps G and U (moe_expert_mlp_save + moe_backward_saved)
    wl.config("tiny", name="graph_saved", T=300, H=320, I=192, E=5, k=3, seed=45, backward=True,
              save_activations=True),
    wl.config("tiny", name="graph_saved_relu2", T=300, H=320, I=192, E=5, k=3, seed=46, backward=True,
              activation="relu2", save_activations=True),
]


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_graph_replays_match_eager(cfg):
    from grouped_gemm_router_amd.layer import MoELayer
    _say("graph", cfg)
    W = {n: device_weights(cfg, n) for n in cfg.mats}
    layer = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.dtype, activation=cfg.activation,
                     save_activations=cfg.save_activations).load_weights(W.get("gate"), W["up"], W["down"])
    logits = torch.from_numpy(wl.make_logits(cfg)).cuda()
    X = to_dev(wl.make_x(cfg))
    dY = to_dev(wl.make_dy(cfg)) if cfg.backward else None
    other = dataclasses.replace(cfg, seed=cfg.seed + 100)
    logits2 = torch.from_numpy(wl.make_logits(other)).cuda()
    X2 = to_dev(wl.make_x(other))

    def step(lg, x):
        y = layer.forward(lg, x, backward_plan=cfg.backward)
        outs = [y]
        if cfg.backward:
            outs += list(layer.backward(x, dY)) + [layer.route_backward(cfg.T)]
        return outs

    def snapshot(outs):
        return [to_bits(t).copy() if t.dtype == torch.bfloat16 else t.cpu().numpy().view(np.int32).copy()
                for t in outs if t is not None]

    eager = snapshot(step(logits, X))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(logits, X)                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step(logits, X)
    torch.cuda.synchronize()
    for rep in range(3):
        step(logits2, X2)                                 # eager work on other inputs, same buffers
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot(outs)
        for i, (a, b) in enumerate(zip(got, eager)):
            assert np.array_equal(a, b), f"replay {rep}: output {i} differs from the eager run"
    # the replayed result against the oracle
    fn = lambda n: host_weight_fn(cfg, n)
    lg, xb = wl.make_logits(cfg), wl.make_x(cfg)
    idx, w, off, h, O, Y, amb_O, amb_Y = oracle_forward(cfg, lg, xb, fn)
    assert np.array_equal(layer.plan(cfg.T, cfg.backward)["topk_idx"].cpu().numpy(), idx)
    assert np.array_equal(layer.plan(cfg.T, cfg.backward)["offsets"].cpu().numpy(), off)
    check_close(orc.bf16_decode(got[0]), Y, "replayed Y", ambiguity=amb_Y)
    if cfg.backward:
        act = cfg.activation
        gated = orc.is_gated(act)
        dy = wl.make_dy(cfg)
        ref = orc.backward(xb, dy, idx, w, fn("gate") if gated else None, fn("up"), fn("down"), E=cfg.E, act=act)
        amb_dwd, amb_dtw = backward_h_ambiguity(cfg, xb, dy, idx, w, fn, act)
        names = ["dX"] + (["dWg"] if gated else []) + ["dWu", "dWd", "d_topk_w", "d_logits"]
        g = dict(zip(names, got[1:]))
        check_close(orc.bf16_decode(g["dX"]), ref["dX"], "replayed dX")
        check_close(g["d_topk_w"].view(np.float32), ref["d_topk_w"], "replayed d_topk_w", ambiguity=amb_dtw,
                    max_rescued=H_RESCUE)
        for key in (("dWg", "dWu", "dWd") if gated else ("dWu", "dWd")):
            gv = orc.bf16_decode(g[key])
            for e in range(cfg.E):
                check_close(gv[e], ref["dW"][key][e], f"replayed {key}[{e}]",
                            ambiguity=amb_dwd.get(e) if key == "dWd" else None, max_rescued=H_RESCUE)
