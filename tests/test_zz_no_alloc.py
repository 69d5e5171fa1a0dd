"""moe_expert_mlp_static: the expert MLP with its workspace in the library's static
per-GPU array, for callers that cannot allocate.  Called through the C ABI, its
outputs equal those of moe_expert_mlp with a caller workspace bit for bit, on two
calls in a row (the second with a smaller input), for the small-token bf16 path
(whose work list lives in the array), the MXFP8 path (X and h codes in the array)
and the row-tile bf16 path (no workspace).  Problems whose workspace exceeds the
array are refused on the host before anything is enqueued."""
import ctypes

import numpy as np
import pytest

from grouped_gemm_router_amd import workloads as wl


def _say(*a):
    print("[case]", *a, flush=True)


def _routed(cfg):
    import torch
    from grouped_gemm_router_amd import binding as B
    logits = torch.from_numpy(wl.make_logits(cfg)).cuda()
    idx, _ = B.route(logits, cfg.k)
    offsets, row_token, _, _ = B.dispatch(idx, cfg.E)
    return offsets, row_token


# (first call, second smaller call) per path
PAIRS = [
    (wl.config("tiny", name="static_decode", T=48, H=256, I=128, E=64, k=4, seed=81),
     wl.config("tiny", name="static_decode", T=20, H=256, I=128, E=64, k=4, seed=82)),
    (wl.config("tiny", name="static_mx", T=96, H=256, I=128, E=6, k=2, dtype="mxfp8", seed=83),
     wl.config("tiny", name="static_mx", T=40, H=256, I=128, E=6, k=2, dtype="mxfp8", seed=84)),
    (wl.config("tiny", name="static_rows", T=300, H=320, I=192, E=5, k=3, seed=85),
     wl.config("tiny", name="static_rows", T=100, H=320, I=192, E=5, k=3, seed=86)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("pair", PAIRS, ids=[p[0].name for p in PAIRS])
def test_static_workspace_matches_caller_workspace(pair):
    import torch
    from grouped_gemm_router_amd import binding as B
    from gpu_helpers import device_weights, to_bits, to_dev
    cfg0 = pair[0]
    W = {n: device_weights(cfg0, n) for n in cfg0.mats}
    Wt = {n: B.pack_weights(W[n]) for n in cfg0.mats}
    scales = None
    if cfg0.dtype == "mxfp8":
        q = {n: B.mx_quantize(Wt[n]) for n in cfg0.mats}
        Wt = {n: q[n][0] for n in cfg0.mats}
        scales = tuple(q[n][1] for n in ("gate", "up", "down"))
    for cfg in pair:
        _say("static workspace", cfg)
        offsets, row_token = _routed(cfg)
        X = to_dev(wl.make_x(cfg))
        ref = B.expert_mlp(X, row_token, offsets, Wt["gate"], Wt["up"], Wt["down"], cfg.k, scales=scales)
        got_h = torch.full((cfg.A, cfg.I), float("nan"), dtype=torch.bfloat16, device="cuda")
        got_o = torch.full((cfg.A, cfg.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        B.expert_mlp(X, row_token, offsets, Wt["gate"], Wt["up"], Wt["down"], cfg.k, scales=scales,
                     H_rows=got_h, O_rows=got_o, static_ws=True)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(got_h), to_bits(ref[0])), "h differs from moe_expert_mlp's"
        assert np.array_equal(to_bits(got_o), to_bits(ref[1])), "O differs from moe_expert_mlp's"


def test_static_workspace_refuses_large_problems_before_launch():
    """A problem whose workspace exceeds MOE_STATIC_SCRATCH_BYTES (8 MiB) gives MOE_ERR_WORKSPACE on
    the host (no device needed); every bf16 problem fits."""
    from grouped_gemm_router_amd import binding as B
    lib = B.lib
    v = ctypes.c_void_p(16)
    limit = 8 << 20
    big = B.problem(8192, 4096, 1024, 512, 10, "mxfp8")
    assert B.workspace_size(big, B.CALL_EXPERT_MLP) > limit
    assert lib.moe_expert_mlp_static(ctypes.byref(big), v, v, v, v, v, v, v, v, v, v, v, None) == 3
    small = B.problem(64, 256, 128, 8, 2, "mxfp8")
    assert B.workspace_size(small, B.CALL_EXPERT_MLP) <= limit
    for p in (B.problem(64, 2048, 512, 1024, 8), B.problem(8192, 4096, 1024, 512, 10)):
        assert B.workspace_size(p, B.CALL_EXPERT_MLP) <= limit
    # argument errors as moe_expert_mlp's
    p = B.problem(64, 256, 128, 8, 2)
    assert lib.moe_expert_mlp_static(ctypes.byref(p), None, None, None, None, None, None, None, None, None,
                                     None, None, None) == 1
    assert lib.moe_expert_mlp_static(ctypes.byref(p), v, v, v, v, v, v, v, v, v, v, v, None) == 1
