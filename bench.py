#!/usr/bin/env python3
"""Benchmark of the routed MoE expert layer on one MI355X.

One step is one pass of the layer's hot path over one batch of synthetic
input: routing, dispatch, the grouped-GEMM expert MLP (gate/up + SwiGLU,
down) and the weighted combine; for the training workload also the backward
(expert MLP and router).
Inputs are resident in HBM before the timed region; weight packing happens at
load time, outside it.

Per workload, three passes over the same steps follow the warmup:
  * the roofline pass: K steps with HIP events around the expert-MLP call (and,
    for training, around the backward call) on the stream its kernels run on,
    giving the calls' average launch durations;
  * the spread pass: K steps with one event between steps (p10 / p50 / p90);
  * the timed region (``ms_per_step``, ``value``): K steps with one timing event
    on each side only (every recorded event leaves the GPU idle for a few
    microseconds, so none sits between the steps), after the two passes above,
    so that it runs at the clocks of a GPU that has been busy for a while.
With --cold-cache a fourth pass reads 512 MiB before every step, which evicts L2
and the Infinity Cache (and leaves clean lines, so the step pays no write-back
of the flush), and times each step on its own (reported under cold_cache).

Prints one JSON line.  Default workload: prefill (T=4096 tokens, hidden 2048,
intermediate 512, 256 experts, top-8, bf16); its line also carries a
``configs`` block with the prefill shape under rank-Zipf routing (every expert
active, non-trivial combine weights), the decode, large MXFP8 and training
workloads, measured the same way (each with its own roofline).  Other workloads (--workload decode
| train | large_mxfp8 | tiny | prefill_rankzipf | model-contract shapes) are for
diagnostics.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "MoE layer fwd/bwd TFLOP/s + tokens/s, % of MFMA (prefill) / HBM (decode) peak"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5033.2       # MI355X dense fp8 / MXFP8 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
FLUSH_BYTES = 512 << 20        # read before each cold-cache step: more than L2 (8 x 4 MB) + Infinity Cache (256 MB)
EXTRA_CONFIGS = ("prefill_rankzipf", "decode", "large_mxfp8", "train", "train_saved")


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cold-cache", action="store_true",
                    help="also time steps after reading 512 MiB (L2 and Infinity Cache evicted), each step alone")
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--tokens", type=int, default=None, help="override the workload's token count T (sweeps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="prefill only: leave out the decode / large MXFP8 / training block")
    ap.add_argument("--graph", action="store_true", help="replay each step from a captured HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before the warmup, copy 1 GiB device to device three times (the known-size "
                         "reference that scales the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args(argv)


def recorded_traffic(workload):
    """HBM bytes of one moe_expert_mlp call from the committed counter runs, or None when there are
    none for this workload or the library sources changed since they were taken."""
    import bench_tools as bt
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha") != bt.source_hash(workload):
        return None
    return int(rec["traffic_bytes"])


def device_weights(cfg, name, experts=None, device_draw=False):
    """All experts' [E, K, N] bf16 weights on the device (experts not listed hold NaN).  Below 2^31
    elements they are the seeded numpy draws the tests use, unless ``device_draw``; larger sets (the
    big expert shapes) and device draws come from a seeded torch generator on the device, N(0, 1/K)
    like the numpy ones, because the host draw would take minutes.  Timing does not depend on the
    values."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    from grouped_gemm_router_amd import workloads as wl
    K, N = wl.weight_shape(cfg, name)
    out = torch.full((cfg.E, K, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    todo = range(cfg.E) if experts is None else sorted(set(int(e) for e in experts))
    if device_draw or cfg.E * K * N >= 2 ** 31:
        g = torch.Generator(device="cuda")
        g.manual_seed(cfg.seed * 16 + ("gate", "up", "down").index(name))
        for e in todo:
            out[e].copy_(torch.randn((K, N), generator=g, device="cuda").mul_(K ** -0.5))
        return out
    with ThreadPoolExecutor(16) as ex:
        for e, bits in ex.map(lambda e: (e, wl.make_expert_weight(cfg, name, e)), todo):
            out[e].copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
    return out


def step_flops(cfg, active_rows):
    """Algorithmic FLOP of the expert MLP (2 H I per weight matrix and row) and of its backward
    (dX, the weight gradients and P: 4 H I per matrix and row; the recompute is not counted)."""
    A, H, I, m = active_rows, cfg.H, cfg.I, len(cfg.mats)
    fwd = 2.0 * m * A * H * I
    bwd = 4.0 * m * A * H * I if cfg.backward else 0.0
    return fwd, bwd


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(cfg, logits, X, dY, min_s=10.0, max_reps=20):
    """The oracle, as it stands, on the host cores: routing and dispatch of all
    tokens plus the expert MLP and combine (and backward for training) of a
    fixed sample of tokens, repeated until about ``min_s`` seconds.  The seeded
    weights the sample needs are drawn before the timed region."""
    from threadpoolctl import threadpool_info
    from oracle import moe_oracle as orc
    from grouped_gemm_router_amd import workloads as wl
    cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    ntok = {"prefill": cfg.T, "decode": cfg.T, "tiny": cfg.T, "prefill_rankzipf": 1024,
            "large_mxfp8": 128, "train": 16, "train_saved": 16}.get(cfg.name, 64)
    if cfg.H * cfg.I >= 4096 * 2048:
        ntok = 2          # the large expert shapes: each sampled expert's weights take seconds to draw
    ntok = min(ntok, cfg.T)
    toks = np.sort(np.random.default_rng(0).choice(cfg.T, ntok, replace=False))
    idx, w = orc.route(logits, cfg.k)
    cache = {(n, int(e)): wl.make_expert_weight(cfg, n, int(e))
             for n in cfg.mats for e in np.unique(idx[toks])}
    fn = lambda n: (lambda e: cache[(n, int(e))]) if n in cfg.mats else None
    reps, t_route, t_mlp = 0, 0.0, 0.0
    while reps < max_reps and (t_route + t_mlp) < min_s:
        t0 = time.perf_counter()
        idx, w = orc.route(logits, cfg.k)
        orc.dispatch(idx, cfg.E)
        t1 = time.perf_counter()
        orc.layer_forward_tokens(X, idx, w, fn("gate"), fn("up"), fn("down"), toks, mxfp8=cfg.dtype == "mxfp8",
                                 act=cfg.activation, limit=cfg.act_limit or None)
        if cfg.backward:
            orc.backward_tokens(X, dY, idx, w, fn("gate"), fn("up"), fn("down"), toks,
                                act=cfg.activation, limit=cfg.act_limit or None)
        t2 = time.perf_counter()
        t_route += t1 - t0
        t_mlp += t2 - t1
        reps += 1
    t_route /= reps
    t_mlp /= reps
    f_fwd, f_bwd = step_flops(cfg, ntok * cfg.k)
    return {"value": round((f_fwd + f_bwd) / t_mlp / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "cpu_model": cpu_model(), "kind": "oracle",
            "tokens_per_s": round(ntok / (t_mlp + t_route * ntok / cfg.T), 2),
            "sample": f"float64 numpy oracle, mean of {reps} runs: routing+dispatch of all {cfg.T} tokens "
                      f"({t_route:.3f} s) and the expert MLP + combine{' + backward' if cfg.backward else ''} "
                      f"of {ntok} sampled tokens ({t_mlp:.3f} s); TFLOP/s counts the sampled tokens' work"}


def _roofline(kernel, flops, nbytes, ms, peak_tflops, traffic=None):
    """Roofline of one call: the bound is the roofline with the longer time at peak."""
    if nbytes / (PEAK_HBM_GBPS * 1e9) > flops / (peak_tflops * 1e12):
        achieved = nbytes / (ms * 1e-3) / 1e9
        return {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                "avg_launch_ms": round(ms, 5)}
    achieved = flops / (ms * 1e-3) / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak_tflops,
            "unit": "TFLOP/s", "frac": round(achieved / peak_tflops, 4), "traffic": traffic,
            "avg_launch_ms": round(ms, 5)}


def measure(cfg, args, device_draw=False):
    """Runs the workload (warmup, timed region, roofline pass, spread pass, optional cold-cache
    pass) and returns its record; ``_inputs`` holds the host inputs for the CPU baseline."""
    import torch
    from grouped_gemm_router_amd import workloads as wl
    from grouped_gemm_router_amd.layer import MoELayer

    logits_np, X_np = wl.make_logits(cfg), wl.make_x(cfg)
    dY_np = wl.make_dy(cfg) if cfg.backward else None
    full_weights = cfg.E * cfg.H * cfg.I <= 128 * 4096 * 1024
    experts = None
    if not full_weights:
        # too large to draw every expert quickly: only the experts the router picks get weights, the
        # others hold NaN (never read by the layer)
        from grouped_gemm_router_amd import binding as B
        idx, _ = B.route(torch.from_numpy(logits_np).cuda(), cfg.k)
        experts = torch.unique(idx).cpu().numpy()
    W = {n: device_weights(cfg, n, experts, device_draw) for n in cfg.mats}
    logits = torch.from_numpy(logits_np).cuda()
    X = torch.from_numpy(X_np.view(np.int16)).cuda().view(torch.bfloat16)
    dY = torch.from_numpy(dY_np.view(np.int16)).cuda().view(torch.bfloat16) if cfg.backward else None
    layer = MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, cfg.dtype, activation=cfg.activation,
                     act_limit=cfg.act_limit, save_activations=cfg.save_activations).load_weights(
        W.get("gate"), W["up"], W["down"])
    del W
    torch.cuda.synchronize()

    def step(mlp_ev=None, bwd_ev=None):
        layer.forward(logits, X, backward_plan=cfg.backward, mlp_events=mlp_ev)
        if cfg.backward:
            if bwd_ev is not None:
                bwd_ev[0].record()
            layer.backward(X, dY)
            if bwd_ev is not None:
                bwd_ev[1].record()
            layer.route_backward(cfg.T)

    if args.copy_calibration:
        from bench_tools import COPY_BYTES
        src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
    run = graph.replay if graph is not None else step
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # roofline pass: events around the expert-MLP call (and the backward call) of every step
    mlp_ms = bwd_ms = None
    if graph is None:
        mlp_evs = [(ev(), ev()) for _ in range(args.steps)]
        bwd_evs = [(ev(), ev()) for _ in range(args.steps)] if cfg.backward else [None] * args.steps
        for i in range(args.steps):
            step(mlp_evs[i], bwd_evs[i])
        torch.cuda.synchronize()
        mlp_ms = float(np.mean([a.elapsed_time(b) for a, b in mlp_evs]))
        if cfg.backward:
            bwd_ms = float(np.mean([a.elapsed_time(b) for a, b in bwd_evs]))

    # spread pass: one event between steps
    marks = [ev() for _ in range(args.steps + 1)]
    marks[0].record()
    for i in range(args.steps):
        run()
        marks[i + 1].record()
    torch.cuda.synchronize()
    step_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])

    # timed region: K steps, one event on each side
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        run()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_start.elapsed_time(t_end) / args.steps

    cold_ms = None
    if args.cold_cache:
        # 512 MiB read before each step (its lines replace everything cached), each step timed alone
        flush = torch.full((FLUSH_BYTES // 4,), 1.0, dtype=torch.float32, device="cuda")
        n_cold = min(args.steps, 20)
        cold = [(ev(), ev()) for _ in range(n_cold)]
        for i in range(n_cold):
            torch.amax(flush)
            cold[i][0].record()
            run()
            cold[i][1].record()
        torch.cuda.synchronize()
        cold_ms = np.array([a.elapsed_time(b) for a, b in cold])
        del flush

    pl = layer.plan(cfg.T, cfg.backward)
    n_active = int(np.count_nonzero(np.diff(pl["offsets"].cpu().numpy())))
    del layer, pl
    torch.cuda.empty_cache()

    f_fwd, f_bwd = step_flops(cfg, cfg.A)
    tflops = (f_fwd + f_bwd) / (ms * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if cfg.dtype == "mxfp8" else PEAK_BF16_TFLOPS
    wbytes = 1 if cfg.dtype == "mxfp8" else 2
    weight_bytes = n_active * len(cfg.mats) * cfg.H * cfg.I * wbytes
    act_bytes = cfg.T * cfg.E * 4 + cfg.T * cfg.H * 2 * 2          # logits, X, Y
    if cfg.backward:
        # dY and dX, the weight gradients of the active experts, d_topk_w and d_logits
        act_bytes += cfg.T * cfg.H * 2 * 2 + n_active * len(cfg.mats) * cfg.H * cfg.I * 2 + cfg.T * cfg.E * 4
    rec = {
        "workload": cfg.name, "T": cfg.T, "hidden": cfg.H, "intermediate": cfg.I, "experts": cfg.E,
        "top_k": cfg.k, "active_experts": n_active, "backward": cfg.backward,
        "saved_activations": cfg.save_activations,
        "activation": cfg.activation if not cfg.act_limit else f"{cfg.activation}({cfg.act_limit:g})",
        "dtype": "mxfp8" if cfg.dtype == "mxfp8" else "bf16",
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "value": round(tflops, 3), "unit": "TFLOP/s",
        "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
        "frac_of_mfma_peak": round(tflops / peak, 4),
        "hbm_GBps_algorithmic": round((weight_bytes + act_bytes) / (ms * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round((weight_bytes + act_bytes) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "algorithmic_bytes": int(weight_bytes + act_bytes),
        "wall_s_timed_region": round(wall, 4),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 5) for q in (10, 50, 90)],
        "graph": bool(args.graph),
        "_inputs": (logits_np, X_np, dY_np),
    }
    if cold_ms is not None:
        rec["cold_cache"] = {"flush_bytes": FLUSH_BYTES, "steps": int(cold_ms.size),
                             "step_ms_p10_p50_p90": [round(float(np.percentile(cold_ms, q)), 5) for q in (10, 50, 90)],
                             "value_at_p50": round((f_fwd + f_bwd) / (float(np.median(cold_ms)) * 1e-3) / 1e12, 3)}
    if mlp_ms is not None:
        # algorithmic bytes of one expert-MLP call: the active experts' weights once, X rows in and
        # h rows out (gate/up), h rows in and O rows out (down)
        mlp_bytes = weight_bytes + cfg.A * (cfg.H + cfg.I) * 2 * 2
        rec["roofline"] = _roofline("moe_expert_mlp (gate/up+activation and down grouped GEMMs)", f_fwd,
                                    mlp_bytes, mlp_ms, peak, recorded_traffic(cfg.name))
    if bwd_ms is not None:
        # algorithmic bytes of one backward call: dY and X rows, the weights, h (recomputed) and the
        # weight gradients of the active experts, dX
        bwd_bytes = 2 * weight_bytes + cfg.T * cfg.H * 2 * 3
        name = ("moe_backward_saved (P, elementwise pass over the saved G and U, dX rows, token reduce, "
                "weight gradients)" if cfg.save_activations else
                "moe_backward (P, recompute, dX rows, token reduce, weight gradients)")
        rec["backward_roofline"] = _roofline(name, f_bwd, bwd_bytes, bwd_ms, peak)
    return rec


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the layer runs every "
              "expert on one MI355X; see the design notes for how it would shard).", file=sys.stderr)
        return 2
    from grouped_gemm_router_amd import workloads as wl

    cfg = wl.config(args.workload) if args.tokens is None else wl.config(args.workload, T=args.tokens)
    rec = measure(cfg, args)
    logits_np, X_np, dY_np = rec.pop("_inputs")
    out = {
        "metric": METRIC,
        "value": rec["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec["dtype"],
        "data": "synthetic (seeded numpy draws; shapes and routing skew of the workload)",
        "config": {k: rec[k] for k in ("workload", "T", "hidden", "intermediate", "experts", "top_k",
                                       "active_experts", "backward", "activation", "graph")},
    }
    for k in ("tokens_per_s", "frac_of_mfma_peak", "hbm_GBps_algorithmic", "wall_s_timed_region",
              "step_ms_p10_p50_p90", "cold_cache", "roofline", "backward_roofline"):
        if k in rec:
            out[k] = rec[k]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, logits_np, X_np, dY_np)
    del logits_np, X_np, dY_np
    if args.workload == "prefill" and args.tokens is None and not args.no_configs:
        # the other workloads, measured the same way, with weights drawn on the device
        configs = {}
        for name in EXTRA_CONFIGS:
            r = measure(wl.config(name), args, device_draw=True)
            r.pop("_inputs")
            r.pop("steps")
            r.pop("warmup")
            configs[name] = r
        out["configs"] = configs
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
