"""Helpers shared by the GPU parity tests: moving bf16 bit patterns to and
from the device, device-resident seeded weights, and the tolerance check
|gpu - oracle| <= 1e-2 + 2e-2 * |oracle| (elementwise)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import moe_oracle as orc
from grouped_gemm_router_amd import workloads as wl

ATOL, RTOL = 1e-2, 2e-2
# backward checks: elements that may lie outside the base bound and inside the h-rounding
# allowance (a flipped h rounding moves a dW_down element by ulp(h) |dO|)
H_RESCUE = 1e-3


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return orc.bf16_decode(to_bits(t))
    return t.cpu().numpy().astype(np.float64)


def check_close(gpu, ref, what: str, atol=ATOL, rtol=RTOL, ambiguity=None, max_rescued=None):
    """Elementwise |gpu - ref| <= atol + rtol |ref|.  ``ambiguity`` (same shape)
    widens it where a quantised intermediate has several valid roundings: the
    GPU value must then lie within tolerance of one of the valid results (the
    bound plus one bf16 ulp for the output's own rounding).  With ``max_rescued`` the
    widening may only rescue a few elements: at most that fraction of them (and at
    least 2) may lie outside the base bound, so that a real error cannot hide inside
    it.  The message reports how large the widening is against the base bound."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    base = atol + rtol * np.abs(ref)
    lim = base
    widen_msg = ""
    rescued = 0
    if ambiguity is not None:
        amb = np.asarray(ambiguity, dtype=np.float64)
        widen = np.where(amb > 0, amb + (np.abs(ref) + amb) * 2.0 ** -7, 0.0)
        lim = base + widen
        rescued = int(((err > base) & (err <= lim)).sum())
        ratio = widen / base
        widen_msg = (f"; widened {np.mean(widen > 0):.3f} of the elements by {ratio.mean():.3f} of the base "
                     f"bound on average (max {ratio.max():.3g}); {rescued} inside the widening only")
    bad = err > lim
    rel = err / np.maximum(np.abs(ref), 1e-6)
    msg = (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; max abs err {err.max():.3g}; "
           f"mean_rel {float(np.mean(rel[np.abs(ref) > 1e-3])) if (np.abs(ref) > 1e-3).any() else 0:.3g}"
           + widen_msg)
    assert not bad.any(), msg
    if max_rescued is not None:
        assert rescued <= max(2, int(max_rescued * bad.size)), msg
    return msg


def mx_block_sum_ambiguity(x_rows, wg, wu, wd, act="swiglu", limit=None):
    """Ambiguity of the O rows of x_rows on the MXFP8 path with the hardware's FP8 summation
    taken into account (``orc.mx_block_dot_deviation``): G and U of the gate/up GEMM may lie that
    far from the exact ones, which widens the valid requantisations of h, and the down GEMM's own
    sums move O by its deviation (float64 values in, per element of O out)."""
    gated = orc.is_gated(act)
    G, U, h, _ = orc.expert_forward_rows(x_rows, wg, wu, wd, mxfp8=True, act=act, limit=limit)
    dG = orc.mx_block_dot_deviation(x_rows, wg) if gated else None
    dU = orc.mx_block_dot_deviation(x_rows, wu)
    amb = orc.mx_down_ambiguity(G, U, wd, act, limit, dG=dG, dU=dU)
    return amb + np.abs(orc.mx_block_dot_deviation(h, wd))


def check_close_mx(gpu, ref, what, ambiguity, refine_rows, max_rows=0.001):
    """check_close with the MXFP8 requantisation ambiguity, where rows holding an element outside
    it get the ambiguity ``refine_rows(rows)`` returns (``mx_block_sum_ambiguity``: that of an
    implementation on the hardware's FP8 block summation); at most a fraction ``max_rows`` of the
    rows (and at least 2) may need it.  Returns the ambiguity used."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    amb = np.array(ambiguity, dtype=np.float64)
    err = np.abs(gpu - ref)
    lim = ATOL + RTOL * np.abs(ref) + np.where(amb > 0, amb + (np.abs(ref) + amb) * 2.0 ** -7, 0.0)
    rows = np.unique(np.nonzero(err > lim)[0])
    note = ""
    if rows.size:
        assert rows.size <= max(2, int(max_rows * gpu.shape[0])), \
            f"{what}: {rows.size} rows outside the requantisation ambiguity"
        amb[rows] = np.maximum(amb[rows], refine_rows(rows))
        note = f" ({rows.size} rows with the FP8 block-sum ambiguity)"
    check_close(gpu, ref, what + note, ambiguity=amb)
    return amb


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


def oracle_forward(cfg, logits, X, wfn):
    """The oracle's forward of a workload: (topk_idx, topk_w, offsets, h, O, Y, amb_O, amb_Y); the
    ambiguities (MXFP8 only, else None) are what valid alternative roundings of the requantised h
    can change (``mx_down_ambiguity``).  wfn(name) gives the per-expert weight getter."""
    act, lim = cfg.activation, cfg.act_limit or None
    gated = orc.is_gated(act)
    idx, w = orc.route(logits, cfg.k)
    off, row_token, row_slot, slot_row = orc.dispatch(idx, cfg.E)
    mx = cfg.dtype == "mxfp8"
    h, O = orc.expert_mlp(X, row_token, off, wfn("gate") if gated else None, wfn("up"), wfn("down"), mxfp8=mx,
                          act=act, limit=lim)
    amb_O = amb_Y = None
    if mx:
        Xv = orc.bf16_decode(X)
        amb_O = np.zeros_like(O)
        for e in range(cfg.E):
            lo, hi = off[e], off[e + 1]
            if hi > lo:
                wg = orc.bf16_decode(wfn("gate")(e)) if gated else None
                G, U, _, _ = orc.expert_forward_rows(Xv[row_token[lo:hi]], wg, orc.bf16_decode(wfn("up")(e)),
                                                     orc.bf16_decode(wfn("down")(e)), mxfp8=True, act=act, limit=lim)
                amb_O[lo:hi] = orc.mx_down_ambiguity(G, U, orc.bf16_decode(wfn("down")(e)), act=act, limit=lim)
        amb_Y = sum(w[:, j:j + 1] * amb_O[slot_row.reshape(-1, cfg.k)[:, j]] for j in range(cfg.k))
    return idx, w, off, h, O, orc.combine(O, slot_row, w), amb_O, amb_Y


def backward_h_ambiguity(cfg, X, dY, idx, w, fn, act="swiglu", limit=None, experts=None):
    """What other valid bf16 roundings of h = bf16(f(G, U)) can change (``bf16_round_delta``:
    h is a rounding decision on a value the GPU knows to fp32): per expert |delta h|^T |dO|
    with the exact dO = w dY (dW_down), per slot sum_i |delta h_i| |P_i| (d_topk_w)."""
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
        dO = w.reshape(-1)[sl][:, None] * dYv[tok]
        amb_dwd[e] = dh.T @ np.abs(dO)
        amb_dtw.reshape(-1)[sl] = (dh * np.abs(dYv[tok] @ wd.T)).sum(axis=1)
    return amb_dwd, amb_dtw
