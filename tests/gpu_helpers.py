"""Helpers shared by the GPU parity tests: moving bf16 bit patterns to and
from the device, device-resident seeded weights, and the tolerance check
|gpu - oracle| <= 1e-2 + 2e-2 * |oracle| (elementwise)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import moe_oracle as orc
from grouped_gemm_router_amd import workloads as wl

ATOL, RTOL = 1e-2, 2e-2


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return orc.bf16_decode(to_bits(t))
    return t.cpu().numpy().astype(np.float64)


def check_close(gpu, ref, what: str, atol=ATOL, rtol=RTOL, ambiguity=None):
    """Elementwise |gpu - ref| <= atol + rtol |ref|.  ``ambiguity`` (same shape)
    widens it where a quantised intermediate has several valid roundings: the
    GPU value must then lie within tolerance of one of the valid results (the
    bound plus one bf16 ulp for the output's own rounding)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    lim = atol + rtol * np.abs(ref)
    if ambiguity is not None:
        amb = np.asarray(ambiguity, dtype=np.float64)
        lim = lim + np.where(amb > 0, amb + (np.abs(ref) + amb) * 2.0 ** -7, 0.0)
    bad = err > lim
    rel = err / np.maximum(np.abs(ref), 1e-6)
    msg = (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; max abs err {err.max():.3g}; "
           f"mean_rel {float(np.mean(rel[np.abs(ref) > 1e-3])) if (np.abs(ref) > 1e-3).any() else 0:.3g}")
    assert not bad.any(), msg
    return msg


def device_weights(cfg, name, experts=None, fill=float("nan")):
    """[E, K, N] bf16 device tensor with the seeded weights of ``experts`` (all
    when None); the others hold ``fill`` (NaN: an unread expert stays unread)."""
    K, N = wl.weight_shape(cfg, name)
    out = torch.full((cfg.E, K, N), fill, dtype=torch.bfloat16, device="cuda")
    todo = range(cfg.E) if experts is None else sorted(set(int(e) for e in experts))

    def one(e):
        return e, wl.make_expert_weight(cfg, name, e)

    with ThreadPoolExecutor(8) as ex:
        for e, bits in ex.map(one, todo):
            out[e].copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
    return out


def host_weight_fn(cfg, name):
    """Per-expert weight getter for the oracle (regenerates the seeded draw)."""
    return lambda e: wl.make_expert_weight(cfg, name, e)


def backward_h_ambiguity(cfg, X, dY, idx, w, fn, act="swiglu", limit=None, experts=None):
    """What other valid bf16 roundings of h = bf16(f(G, U)) and dO = bf16(w dY) can change
    (``bf16_round_delta``; both are rounding decisions on values the GPU knows to fp32):
    per expert |delta h|^T |dO| + |h|^T |delta dO| (dW_down), per slot
    sum_i |delta h_i| |P_i| (d_topk_w)."""
    off, row_token, row_slot, _ = orc.dispatch(idx, cfg.E)
    Xv, dYv = orc.bf16_decode(X), orc.bf16_decode(dY)
    amb_dwd = {}
    amb_dtw = np.zeros(idx.shape)
    for e in (range(cfg.E) if experts is None else experts):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        tok, sl = row_token[lo:hi], row_slot[lo:hi]
        wg = orc.bf16_decode(fn("gate")(e)) if orc.is_gated(act) else None
        wu, wd = (orc.bf16_decode(fn(n)(e)) for n in ("up", "down"))
        dh = orc.h_ambiguity_rows(Xv[tok], wg, wu, act, limit)
        _, _, h, _ = orc.expert_forward_rows(Xv[tok], wg, wu, wd, act=act, limit=limit)
        dO_exact = w.reshape(-1)[sl][:, None] * dYv[tok]
        dO = orc.bf16_round(dO_exact)
        amb_dwd[e] = dh.T @ np.abs(dO) + np.abs(h).T @ orc.bf16_round_delta(dO_exact)
        amb_dtw.reshape(-1)[sl] = (dh * np.abs(dYv[tok] @ wd.T)).sum(axis=1)
    return amb_dwd, amb_dtw
