"""GPU parity of every call against the CPU oracle on small and ragged
problems (several tiles, partial tiles, empty experts, degenerate k and E),
plus determinism and NaN-poisoned unused experts.  Integer outputs must match
bit for bit; floating-point outputs within 1e-2 + 2e-2*|oracle|."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc
from grouped_gemm_router_amd import workloads as wl

from gpu_helpers import (H_RESCUE, backward_h_ambiguity, check_close, device_weights, host_weight_fn,
                         oracle_forward, to_bits, to_dev, to_f64)

pytestmark = pytest.mark.gpu


def _B():
    from grouped_gemm_router_amd import binding
    return binding


def _say(*a):
    print("[case]", *a, flush=True)


# ------------------------------------------------------------------------------------------
# bf16 rounding of the device conversion (combine with exact products)
# ------------------------------------------------------------------------------------------
def test_combine_rounds_to_nearest_even():
    B = _B()
    _say("combine rounding")
    rng = np.random.default_rng(0)
    T, H = 512, 256
    O = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    for wv in (1 + 2.0 ** -9, 1 - 2.0 ** -9, 1 + 3 * 2.0 ** -9, 0.5 + 2.0 ** -10):
        w = np.full((T, 1), wv, np.float32)
        Y = B.combine(to_dev(O), torch.arange(T, dtype=torch.int32, device="cuda"), torch.from_numpy(w).cuda())
        ref = orc.bf16_encode(orc.bf16_decode(O) * float(np.float32(wv)))
        assert np.array_equal(to_bits(Y), ref)


# ------------------------------------------------------------------------------------------
# routing and dispatch: bit-exact on every workload's logits
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "prefill", "decode", "large_mxfp8", "train", "prefill_rankzipf"])
def test_route_and_dispatch_bit_exact(name):
    B = _B()
    cfg = wl.config(name)
    _say("route/dispatch", name)
    logits = wl.make_logits(cfg)
    idx, w = B.route(torch.from_numpy(logits).cuda(), cfg.k)
    ridx, rw = orc.route(logits, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    wg = w.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(wg - rw) <= 1e-6 + 1e-5 * np.abs(rw))
    got = B.dispatch(idx, cfg.E)
    ref = orc.dispatch(ridx, cfg.E)
    for g, r, n in zip(got, ref, ("offsets", "row_token", "row_slot", "slot_row")):
        assert np.array_equal(g.cpu().numpy(), r), n


@pytest.mark.parametrize("name,T,E,k", [("tiny", 64, 8, 2), ("decode", 32, 256, 8), ("decode", 512, 256, 8),
                                         ("decode", 513, 256, 8), ("large_mxfp8", 409, 512, 10),
                                         ("ties", 97, 1024, 32), ("ties", 1, 3, 3), ("ties", 200, 100, 5),
                                         ("ties", 1030, 96, 7), ("ties", 1024, 5, 5), ("ties", 2050, 256, 16),
                                         ("ties", 1100, 200, 17), ("ties", 1500, 300, 20),
                                         ("ties", 1200, 700, 9)])
def test_route_dispatch_shapes_bit_exact(name, T, E, k):
    """Every logits-per-lane width of the router (E up to 64, 128, 256, 512,
    1024) with whole-wave token groups (T < 1024), and from 1024 tokens on the
    16-lane groups (E <= 256, k <= 16: 1, 8 and 16 logits per lane, a partial
    last wave at T = 1030), 32-lane groups (k > 16 or E > 256) and whole waves
    (E > 512); both dispatch paths: one workgroup for T*k <= 4096, two-stage
    otherwise (with 1 to 32 threads per expert in its count sums)."""
    B = _B()
    _say("route+dispatch", name, T, E, k)
    if name == "ties":
        logits = np.random.default_rng(T).integers(-3, 4, (T, E)).astype(np.float32)
        logits[0, ::3] = -0.0
    else:
        cfg = wl.config(name)
        logits = np.ascontiguousarray(wl.make_logits(cfg)[:T, :E]) if T <= cfg.T else \
            np.random.default_rng(T).standard_normal((T, E)).astype(np.float32)
    idx, w = B.route(torch.from_numpy(logits).cuda(), k)
    ridx, rw = orc.route(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.all(np.abs(w.cpu().numpy().astype(np.float64) - rw) <= 1e-6 + 1e-5 * np.abs(rw))
    got = B.dispatch(idx, E)
    ref = orc.dispatch(ridx, E)
    for g, r, n in zip(got, ref, ("offsets", "row_token", "row_slot", "slot_row")):
        assert np.array_equal(g.cpu().numpy(), r), n


def test_route_ties_and_signed_zeros():
    B = _B()
    _say("route ties")
    T, E, k = 64, 96, 7
    rng = np.random.default_rng(1)
    logits = rng.integers(-2, 3, (T, E)).astype(np.float32)   # many exact ties
    logits[0] = 0.0
    logits[1] = -0.0
    logits[2, ::2] = -0.0
    logits[3] = np.float32(-3.5)
    idx, w = B.route(torch.from_numpy(logits).cuda(), k)
    ridx, rw = orc.route(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.all(np.abs(w.cpu().numpy() - rw) <= 1e-6 + 1e-5 * rw)
    assert np.all(w.cpu().numpy()[0] == np.float32(1.0 / k))


# (the one-workgroup dispatch holds 1, 2 or 4 groups of 64 slots per wave: T k = 1024 | 1032 and
# 2048 | 2056 sit on both sides of its two boundaries)
@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (1, 8, 8), (5, 3, 3), (3000, 7, 2), (9000, 1024, 32),
                                   (4097, 64, 1), (0, 16, 4), (128, 64, 8), (129, 64, 8), (256, 32, 8),
                                   (257, 32, 8)])
def test_dispatch_edge_cases(T, E, k):
    B = _B()
    _say("dispatch", T, E, k)
    rng = np.random.default_rng(T + E + k)
    logits = rng.standard_normal((max(T, 1), E)).astype(np.float32)[:T]
    ridx, _ = orc.route(logits, k) if T else (np.zeros((0, k), np.int32), None)
    idx = torch.from_numpy(np.ascontiguousarray(ridx)).cuda()
    got = B.dispatch(idx, E)
    ref = orc.dispatch(ridx, E)
    for g, r in zip(got, ref):
        assert np.array_equal(g.cpu().numpy(), r)


# ------------------------------------------------------------------------------------------
# packing and MXFP8 quantisation: bit-exact
# ------------------------------------------------------------------------------------------
def test_pack_weights_is_transpose():
    B = _B()
    _say("pack")
    rng = np.random.default_rng(2)
    W = wl.f32_to_bf16_bits(rng.standard_normal((3, 192, 320)).astype(np.float32))
    Wt = B.pack_weights(to_dev(W))
    assert np.array_equal(to_bits(Wt), np.ascontiguousarray(W.transpose(0, 2, 1)))


def test_mx_quantize_bit_exact():
    B = _B()
    _say("mx quantize")
    rng = np.random.default_rng(3)
    x = wl.f32_to_bf16_bits((rng.standard_normal((257, 512)) * 10.0 ** rng.integers(-8, 8, (257, 1))).astype(np.float32))
    x[5, 64:96] = 0                                    # all-zero block
    x[6, :32] = 0x8000                                 # all -0.0
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    allbits = allbits[np.isfinite(orc.bf16_decode(allbits))]
    allbits = allbits[: allbits.size // 32 * 32].reshape(-1, 32)
    for arr in (x, allbits, np.ascontiguousarray(allbits[:, ::-1])):
        q, s = B.mx_quantize(to_dev(arr))
        rq, rs = orc.mx_quantize(orc.bf16_decode(arr))
        assert np.array_equal(s.cpu().numpy(), rs)
        assert np.array_equal(q.cpu().numpy(), rq)


# ------------------------------------------------------------------------------------------
# router backward
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (32, 256, 8), (409, 512, 10), (40, 6, 6), (97, 1024, 32),
                                   (5, 64, 1), (130, 100, 7)])
def test_route_backward_vs_oracle(T, E, k):
    """The kernel on the oracle's inputs: d_topk_w drawn here, the same array for both sides."""
    B = _B()
    _say("route backward", T, E, k)
    rng = np.random.default_rng(T * 7 + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    dw = (rng.standard_normal((T, k)) * 10.0).astype(np.float32)
    idx, w = B.route(torch.from_numpy(logits).cuda(), k)
    dl = B.route_backward(idx, w, torch.from_numpy(dw).cuda(), E)
    dl2 = B.route_backward(idx, w, torch.from_numpy(dw).cuda(), E)
    torch.cuda.synchronize()
    ref = orc.route_backward(logits, k, dw.astype(np.float64))
    got = dl.cpu().numpy().astype(np.float64)
    # fp32 arithmetic on fp32 inputs: a few ulps of the row's largest term
    scale = np.abs(dw).max(axis=1, keepdims=True)
    assert np.all(np.abs(got - ref) <= 1e-5 * scale + 1e-5 * np.abs(ref)), np.abs(got - ref).max()
    assert np.array_equal(got == 0, ref == 0)            # unchosen logits are exactly zero
    assert np.array_equal(dl.cpu().numpy().view(np.int32), dl2.cpu().numpy().view(np.int32))


def route_grad_tolerance(w, dw_ref):
    """Bound on d_logits when d_topk_w carries the layer tolerance a + r|ref| (a = 1e-2, r = 2e-2):
    w_j (|delta d_j| + |delta s|) <= w_j (2a + 2r max_i |d_i|)."""
    return w * (2e-2 + 4e-2 * np.abs(dw_ref).max(axis=1, keepdims=True)) + 1e-6


# ------------------------------------------------------------------------------------------
# forward
# ------------------------------------------------------------------------------------------
def _run_forward(cfg, Wg, Wu, Wd, logits, X):
    from grouped_gemm_router_amd.layer import MoELayer
    layer = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.dtype).load_weights(Wg, Wu, Wd)
    Y = layer.forward(torch.from_numpy(logits).cuda(), to_dev(X))
    torch.cuda.synchronize()
    return layer, layer.plan(cfg.T)


SMALL = [
    wl.config("tiny"),
    wl.config("tiny", name="ragged", T=300, H=320, I=192, E=5, k=3, seed=11),
    wl.config("tiny", name="one_expert", T=77, E=1, k=1, seed=12),
    wl.config("tiny", name="k_eq_E", T=40, E=6, k=6, seed=13),
    wl.config("tiny", name="many_empty", T=9, E=200, k=2, seed=14),
    wl.config("tiny", name="I64", T=600, H=128, I=64, E=4, k=2, seed=15),
    wl.config("tiny", name="mx_small", T=96, H=256, I=128, E=6, k=2, dtype="mxfp8", seed=16),
    wl.config("tiny", name="mx_ragged", T=333, H=384, I=256, E=5, k=3, dtype="mxfp8", seed=17),
    # small-token streams: 5 k steps of gate/up split 1, 1, 1, 2 over the waves, 3 down steps (an
    # odd count for the two-stage ring), experts of more than 16 rows (several row groups)
    wl.config("tiny", name="decode_ragged", T=64, H=320, I=192, E=16, k=8, seed=18),
    # one gate/up k step: three waves of every workgroup stream nothing
    wl.config("tiny", name="decode_h64", T=33, H=64, I=64, E=8, k=2, seed=19),
    # the most experts the small-token work list holds
    wl.config("tiny", name="decode_e1024", T=16, H=128, I=64, E=1024, k=8, seed=20),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_forward_small_vs_oracle(cfg):
    _say("forward", cfg)
    logits, X = wl.make_logits(cfg), wl.make_x(cfg)
    Wg, Wu, Wd = (device_weights(cfg, n) for n in ("gate", "up", "down"))
    layer, pl = _run_forward(cfg, Wg, Wu, Wd, logits, X)
    idx, w, off, h, O, Y, amb_O, amb_Y = oracle_forward(cfg, logits, X, lambda n: host_weight_fn(cfg, n))
    assert np.array_equal(pl["topk_idx"].cpu().numpy(), idx)
    assert np.array_equal(pl["offsets"].cpu().numpy(), off)
    check_close(to_f64(pl["H_rows"]), h, "h")
    check_close(to_f64(pl["O_rows"]), O, "O", ambiguity=amb_O)
    check_close(to_f64(pl["Y"]), Y, "Y", ambiguity=amb_Y)


# expert sizes that land in every row class of the row-grouped GEMMs (n = q * 256 + r: full
# 256-row tiles and remainders above 192 rows, and one 192-, 128- or 64-row tile for the
# remainders up to 192, 128 and 64 rows), including each class boundary
REMAINDER_COUNTS = [0, 1, 63, 64, 65, 100, 127, 128, 129, 192, 193, 200, 255, 256, 257, 300, 320, 321, 384, 385,
                    448, 449, 513]


def remainder_logits(counts, E, seed):
    """k = 1 logits that send exactly counts[e] tokens to expert e (tokens in a shuffled order)."""
    rng = np.random.default_rng(seed)
    owner = rng.permutation(np.repeat(np.arange(E), counts))
    logits = 0.1 * rng.standard_normal((owner.size, E)).astype(np.float32)
    logits[np.arange(owner.size), owner] = 4.0
    return np.ascontiguousarray(logits)


@pytest.mark.parametrize("act", ["swiglu", "relu2"])
def test_forward_backward_every_row_class(act):
    _say("row classes", act, REMAINDER_COUNTS)
    from grouped_gemm_router_amd.layer import MoELayer
    E = len(REMAINDER_COUNTS)
    logits = remainder_logits(REMAINDER_COUNTS, E, 61)
    cfg = wl.config("tiny", name="row_classes", T=logits.shape[0], H=192, I=128, E=E, k=1, seed=61, backward=True)
    gated = orc.is_gated(act)
    X, dY = wl.make_x(cfg), wl.make_dy(cfg)
    W = {n: device_weights(cfg, n) for n in (("gate", "up", "down") if gated else ("up", "down"))}
    layer = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, activation=act).load_weights(W.get("gate"), W["up"], W["down"])
    layer.forward(torch.from_numpy(logits).cuda(), to_dev(X), backward_plan=True)
    pl = layer.plan(cfg.T, True)
    torch.cuda.synchronize()
    fn = lambda n: host_weight_fn(cfg, n)
    idx, w = orc.route(logits, cfg.k)
    off, row_token, row_slot, slot_row = orc.dispatch(idx, cfg.E)
    h, O = orc.expert_mlp(X, row_token, off, fn("gate") if gated else None, fn("up"), fn("down"), act=act)
    Y = orc.combine(O, slot_row, w)
    assert np.array_equal(np.diff(off), REMAINDER_COUNTS)
    assert np.array_equal(pl["offsets"].cpu().numpy(), off)
    check_close(to_f64(pl["H_rows"]), h, "h")
    check_close(to_f64(pl["O_rows"]), O, "O")
    check_close(to_f64(pl["Y"]), Y, "Y")
    dX, dWg, dWu, dWd, dtw = layer.backward(to_dev(X), to_dev(dY))
    torch.cuda.synchronize()
    ref = orc.backward(X, dY, idx, w, fn("gate") if gated else None, fn("up"), fn("down"), E=cfg.E, act=act)
    amb_dwd, amb_dtw = backward_h_ambiguity(cfg, X, dY, idx, w, fn, act)
    check_close(to_f64(dX), ref["dX"], "dX")
    check_close(dtw.cpu().numpy(), ref["d_topk_w"], "d_topk_w", ambiguity=amb_dtw, max_rescued=H_RESCUE)
    g = {"dWg": to_f64(dWg) if gated else None, "dWu": to_f64(dWu), "dWd": to_f64(dWd)}
    for key in (("dWg", "dWu", "dWd") if gated else ("dWu", "dWd")):
        for e in range(cfg.E):
            check_close(g[key][e], ref["dW"][key][e], f"{key}[{e}] ({REMAINDER_COUNTS[e]} rows)",
                        ambiguity=amb_dwd.get(e) if key == "dWd" else None, max_rescued=H_RESCUE)


ACTS = [("swiglu", 0.0), ("swiglu_clamp", 1.0), ("swiglu_oai", 1.0), ("swiglu_oai", 7.0), ("geglu", 0.0),
        ("reglu", 0.0), ("relu2", 0.0)]
ACT_CFGS = [wl.config("tiny", name="act_rows", T=300, H=320, I=192, E=5, k=3, seed=51),
            wl.config("tiny", name="act_decode", T=24, H=256, I=128, E=16, k=4, seed=52),
            wl.config("tiny", name="act_mx", T=96, H=256, I=128, E=6, k=2, dtype="mxfp8", seed=53)]


@pytest.mark.parametrize("act,limit", ACTS, ids=[f"{a}{l:g}" for a, l in ACTS])
@pytest.mark.parametrize("cfg", ACT_CFGS, ids=[c.name for c in ACT_CFGS])
def test_forward_activations_vs_oracle(cfg, act, limit):
    """Every activation on the three forward paths (row tiles with a remainder,
    small-token weight streaming, MXFP8); clamp 1.0 makes the clamps bind often.  The
    ungated ReLU^2 expert gets no gate weight at all."""
    from grouped_gemm_router_amd.layer import MoELayer
    _say("forward", act, limit, cfg)
    gated = orc.is_gated(act)
    logits, X = wl.make_logits(cfg), wl.make_x(cfg)
    W = {n: device_weights(cfg, n) for n in (("gate", "up", "down") if gated else ("up", "down"))}
    layer = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.dtype, activation=act, act_limit=limit).load_weights(
        W.get("gate"), W["up"], W["down"])
    layer.forward(torch.from_numpy(logits).cuda(), to_dev(X))
    torch.cuda.synchronize()
    pl = layer.plan(cfg.T)
    fn = lambda n: host_weight_fn(cfg, n)
    idx, w = orc.route(logits, cfg.k)
    off, row_token, row_slot, slot_row = orc.dispatch(idx, cfg.E)
    mx = cfg.dtype == "mxfp8"
    lim = limit or None
    h, O = orc.expert_mlp(X, row_token, off, fn("gate") if gated else None, fn("up"), fn("down"), mxfp8=mx, act=act,
                          limit=lim)
    amb_O = None
    if mx:
        Xv = orc.bf16_decode(X)
        amb_O = np.zeros_like(O)
        for e in range(cfg.E):
            lo, hi = off[e], off[e + 1]
            if hi > lo:
                wg = orc.bf16_decode(fn("gate")(e)) if gated else None
                wu, wd = (orc.bf16_decode(fn(n)(e)) for n in ("up", "down"))
                G, U, _, _ = orc.expert_forward_rows(Xv[row_token[lo:hi]], wg, wu, wd, mxfp8=True, act=act,
                                                     limit=lim)
                amb_O[lo:hi] = orc.mx_down_ambiguity(G, U, wd, act=act, limit=lim)
    check_close(to_f64(pl["H_rows"]), h, f"{act} h")
    check_close(to_f64(pl["O_rows"]), O, f"{act} O", ambiguity=amb_O)


@pytest.mark.parametrize("act,limit", ACTS, ids=[f"{a}{l:g}" for a, l in ACTS])
def test_backward_activations_vs_oracle(act, limit):
    from grouped_gemm_router_amd.layer import MoELayer
    cfg = wl.config("tiny", name="act_bwd", T=300, H=320, I=192, E=5, k=3, seed=54, backward=True)
    _say("backward", act, limit, cfg)
    gated = orc.is_gated(act)
    logits, X, dY = wl.make_logits(cfg), wl.make_x(cfg), wl.make_dy(cfg)
    W = {n: device_weights(cfg, n) for n in (("gate", "up", "down") if gated else ("up", "down"))}
    layer = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, activation=act, act_limit=limit).load_weights(
        W.get("gate"), W["up"], W["down"])
    layer.forward(torch.from_numpy(logits).cuda(), to_dev(X), backward_plan=True)
    dX, dWg, dWu, dWd, dtw = layer.backward(to_dev(X), to_dev(dY))
    torch.cuda.synchronize()
    idx, w = orc.route(logits, cfg.k)
    fn = lambda n: host_weight_fn(cfg, n)
    ref = orc.backward(X, dY, idx, w, fn("gate") if gated else None, fn("up"), fn("down"), E=cfg.E, act=act,
                       limit=limit or None)
    amb_dwd, amb_dtw = backward_h_ambiguity(cfg, X, dY, idx, w, fn, act, limit or None)
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


def test_empty_batch_forward_backward():
    """T = 0: every call accepts the empty arrays, the forward produces nothing and the backward
    writes exact zeros to every weight gradient."""
    _say("empty batch")
    from grouped_gemm_router_amd.layer import MoELayer
    cfg = wl.config("tiny", name="empty", T=0, seed=71, backward=True)
    W = {n: device_weights(cfg, n) for n in ("gate", "up", "down")}
    layer = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k).load_weights(W["gate"], W["up"], W["down"])
    logits = torch.zeros(0, cfg.E, dtype=torch.float32, device="cuda")
    X = torch.zeros(0, cfg.H, dtype=torch.bfloat16, device="cuda")
    grads = layer.plan(0, True)["grads"]
    for g in grads[1:4]:
        g.fill_(1.0)                                     # must be overwritten with zeros
    Y = layer.forward(logits, X, backward_plan=True)
    dX, dWg, dWu, dWd, dtw = layer.backward(X, X)
    dlog = layer.route_backward(0)
    torch.cuda.synchronize()
    assert Y.shape == (0, cfg.H) and dX.shape == (0, cfg.H) and dtw.shape == (0, cfg.k) and dlog.shape == (0, cfg.E)
    assert np.array_equal(layer.plan(0, True)["offsets"].cpu().numpy(), np.zeros(cfg.E + 1, np.int32))
    for g in (dWg, dWu, dWd):
        assert not torch.any(g.view(torch.int16) != 0)   # +0.0 bit patterns


def test_forward_deterministic_and_unused_experts_unread():
    _say("determinism + NaN poisoning")
    cfg = wl.config("tiny", name="poison", T=48, H=256, I=128, E=256, k=2, seed=21)
    logits, X = wl.make_logits(cfg), wl.make_x(cfg)
    idx, _ = orc.route(logits, cfg.k)
    active = np.unique(idx)
    assert len(active) < cfg.E
    W_full = [device_weights(cfg, n) for n in ("gate", "up", "down")]
    W_pois = [device_weights(cfg, n, experts=active) for n in ("gate", "up", "down")]
    _, p1 = _run_forward(cfg, *W_full, logits, X)
    y1 = to_bits(p1["Y"]).copy()
    _, p2 = _run_forward(cfg, *W_full, logits, X)
    assert np.array_equal(to_bits(p2["Y"]), y1)
    _, p3 = _run_forward(cfg, *W_pois, logits, X)
    assert np.array_equal(to_bits(p3["Y"]), y1)
    assert np.isfinite(to_f64(p3["Y"])).all()


# ------------------------------------------------------------------------------------------
# backward
# ------------------------------------------------------------------------------------------
BWD = [
    wl.config("tiny", backward=True),
    wl.config("tiny", name="bwd_ragged", T=300, H=320, I=192, E=5, k=3, seed=31, backward=True),
    wl.config("tiny", name="bwd_empty", T=6, H=128, I=64, E=40, k=2, seed=32, backward=True),
    wl.config("tiny", name="bwd_long", T=700, H=256, I=128, E=2, k=1, seed=33, backward=True),
]


@pytest.mark.parametrize("cfg", BWD, ids=[c.name for c in BWD])
def test_backward_small_vs_oracle(cfg):
    _say("backward", cfg)
    from grouped_gemm_router_amd.layer import MoELayer
    logits, X, dY = wl.make_logits(cfg), wl.make_x(cfg), wl.make_dy(cfg)
    W = {n: device_weights(cfg, n) for n in ("gate", "up", "down")}
    layer = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k).load_weights(W["gate"], W["up"], W["down"])
    layer.forward(torch.from_numpy(logits).cuda(), to_dev(X), backward_plan=True)
    dX, dWg, dWu, dWd, dtw = layer.backward(to_dev(X), to_dev(dY))
    torch.cuda.synchronize()
    idx, w = orc.route(logits, cfg.k)
    fn = lambda n: host_weight_fn(cfg, n)
    ref = orc.backward(X, dY, idx, w, fn("gate"), fn("up"), fn("down"), E=cfg.E)
    amb_dwd, amb_dtw = backward_h_ambiguity(cfg, X, dY, idx, w, fn)
    check_close(to_f64(dX), ref["dX"], "dX")
    check_close(dtw.cpu().numpy(), ref["d_topk_w"], "d_topk_w", ambiguity=amb_dtw, max_rescued=H_RESCUE)
    # router backward chained on the layer's d_topk_w, against the oracle's chain
    dlog = layer.route_backward(cfg.T).cpu().numpy().astype(np.float64)
    rdl = orc.route_backward(logits, cfg.k, ref["d_topk_w"])
    lim = np.zeros_like(rdl)
    np.put_along_axis(lim, idx.astype(np.int64), route_grad_tolerance(w, ref["d_topk_w"]), axis=1)
    assert np.all(np.abs(dlog - rdl) <= lim), np.abs(dlog - rdl).max()
    g = {"dWg": to_f64(dWg), "dWu": to_f64(dWu), "dWd": to_f64(dWd)}
    for key in ("dWg", "dWu", "dWd"):
        for e in range(cfg.E):
            check_close(g[key][e], ref["dW"][key][e], f"{key}[{e}]",
                        ambiguity=amb_dwd.get(e) if key == "dWd" else None, max_rescued=H_RESCUE)
    # a second backward gives the same bits (fixed reduction order, no atomics)
    first = [to_bits(t).copy() for t in (dX, dWg, dWu, dWd)] + [dtw.cpu().numpy().copy()]
    layer.backward(to_dev(X), to_dev(dY))
    torch.cuda.synchronize()
    again = [to_bits(t) for t in (dX, dWg, dWu, dWd)] + [dtw.cpu().numpy()]
    for a, b in zip(first, again):
        assert np.array_equal(a, b)
