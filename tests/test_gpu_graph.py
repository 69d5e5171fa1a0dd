"""HIP-graph capture of the layer: a captured forward (and forward + backward)
replayed several times, with eager work on other inputs through the same plan
buffers between the replays, gives the eager result bit for bit every time.
No call of the library allocates or clears memory with a memset, so the whole
step can be captured."""
import dataclasses

import numpy as np
import pytest
import torch

from grouped_gemm_router_amd import workloads as wl

from gpu_helpers import device_weights, to_bits, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    wl.config("tiny", name="graph_rows", T=300, H=320, I=192, E=5, k=3, seed=41, backward=True),
    wl.config("tiny", name="graph_decode", T=24, H=256, I=128, E=64, k=4, seed=42),
    wl.config("tiny", name="graph_mx", T=96, H=256, I=128, E=6, k=2, dtype="mxfp8", seed=43),
    wl.config("tiny", name="graph_relu2", T=300, H=320, I=192, E=5, k=3, seed=44, backward=True, activation="relu2"),
]


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_graph_replays_match_eager(cfg):
    from grouped_gemm_router_amd.layer import MoELayer
    _say("graph", cfg)
    W = {n: device_weights(cfg, n) for n in cfg.mats}
    layer = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.dtype, activation=cfg.activation).load_weights(
        W.get("gate"), W["up"], W["down"], keep_math=cfg.backward)
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
