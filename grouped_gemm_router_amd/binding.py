"""Thin Python binding of libmoe.so (include/moe.h) over ctypes.

Argument marshalling only: every step of the layer runs in the HIP library;
PyTorch supplies device memory and the current HIP stream.  Importing this
module fails loudly when the library has not been built; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_LIBRARY", os.path.join(_PKG, "libmoe.so"))

MOE_OK = 0
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED_SHAPE", 3: "MOE_ERR_WORKSPACE",
          4: "MOE_ERR_UNSUPPORTED_DEVICE", 5: "MOE_ERR_HIP"}
DTYPE = {"bf16": 0, "mxfp8": 1}
ACT = {"swiglu": 0, "swiglu_clamp": 1, "swiglu_oai": 2, "geglu": 3, "reglu": 4, "relu2": 5}
# ReLU^2 experts have no gate weight: every gate argument is None (NULL) for it
UNGATED = ("relu2",)
CALL_DISPATCH, CALL_EXPERT_MLP, CALL_BACKWARD = 0, 1, 2

EXPORTS = ("moe_status_string", "moe_validate_problem", "moe_workspace_size", "moe_check_device",
           "moe_route", "moe_dispatch", "moe_pack_weights", "moe_mx_quantize", "moe_expert_mlp",
           "moe_combine", "moe_backward", "moe_route_backward", "moe_grouped_gemm", "moe_expert_mlp_static",
           "moe_expert_mlp_save", "moe_backward_saved")


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


class moe_problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("act_limit", ctypes.c_float)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m grouped_gemm_router_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    PP = ctypes.POINTER(moe_problem)
    sig = {
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_validate_problem": (ctypes.c_int, [PP]),
        "moe_workspace_size": (ctypes.c_int, [PP, ctypes.c_int, ctypes.POINTER(SZ)]),
        "moe_check_device": (ctypes.c_int, []),
        "moe_route": (ctypes.c_int, [P, I32, I32, I32, P, P, P]),
        "moe_route_backward": (ctypes.c_int, [P, P, P, I32, I32, I32, P, P]),
        "moe_dispatch": (ctypes.c_int, [P, I32, I32, I32, P, P, P, P, P, SZ, P]),
        "moe_pack_weights": (ctypes.c_int, [P, I32, I32, I32, P, P]),
        "moe_mx_quantize": (ctypes.c_int, [P, I64, I32, P, P, P]),
        "moe_expert_mlp": (ctypes.c_int, [PP, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "moe_combine": (ctypes.c_int, [P, P, P, I32, I32, I32, P, P]),
        "moe_backward": (ctypes.c_int, [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "moe_grouped_gemm": (ctypes.c_int, [I32, P, I32, I64, I32, I32, P, P, P, P, P, P]),
        "moe_expert_mlp_static": (ctypes.c_int, [PP, P, P, P, P, P, P, P, P, P, P, P, P]),
        "moe_expert_mlp_save": (ctypes.c_int, [PP, P, P, P, P, P, P, P, P, P, P]),
        "moe_backward_saved": (ctypes.c_int, [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


lib = _load()


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoEError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _expect(t, name, dtype, shape=None):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def problem(T, H, I, E, k, dtype="bf16", activation="swiglu", act_limit=0.0) -> moe_problem:
    return moe_problem(T, H, I, E, k, DTYPE[dtype], ACT[activation], float(act_limit or 0.0))


def validate_problem(p: moe_problem) -> int:
    return lib.moe_validate_problem(ctypes.byref(p))


def workspace_size(p: moe_problem, call: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", lib.moe_workspace_size(ctypes.byref(p), call, ctypes.byref(n)))
    return n.value


def status_string(s: int) -> str:
    return lib.moe_status_string(s).decode()


def _workspace(p, call, device):
    n = workspace_size(p, call)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device), n


def route(logits: torch.Tensor, k: int, topk_idx=None, topk_w=None):
    T, E = logits.shape
    _expect(logits, "logits", torch.float32)
    topk_idx = torch.empty(T, k, dtype=torch.int32, device=logits.device) if topk_idx is None else topk_idx
    topk_w = torch.empty(T, k, dtype=torch.float32, device=logits.device) if topk_w is None else topk_w
    _expect(topk_idx, "topk_idx", torch.int32, (T, k))
    _expect(topk_w, "topk_w", torch.float32, (T, k))
    _check("moe_route", lib.moe_route(_ptr(logits), T, E, k, _ptr(topk_idx), _ptr(topk_w), _stream()))
    return topk_idx, topk_w


def route_backward(topk_idx: torch.Tensor, topk_w: torch.Tensor, d_topk_w: torch.Tensor, E: int, d_logits=None):
    T, k = topk_idx.shape
    _expect(topk_idx, "topk_idx", torch.int32)
    _expect(topk_w, "topk_w", torch.float32, (T, k))
    _expect(d_topk_w, "d_topk_w", torch.float32, (T, k))
    d_logits = torch.empty(T, E, dtype=torch.float32, device=topk_idx.device) if d_logits is None else d_logits
    _expect(d_logits, "d_logits", torch.float32, (T, E))
    _check("moe_route_backward", lib.moe_route_backward(_ptr(topk_idx), _ptr(topk_w), _ptr(d_topk_w), T, E, k,
                                                        _ptr(d_logits), _stream()))
    return d_logits


def dispatch(topk_idx: torch.Tensor, E: int, out=None, ws=None):
    T, k = topk_idx.shape
    _expect(topk_idx, "topk_idx", torch.int32)
    dev = topk_idx.device
    if out is None:
        out = (torch.empty(E + 1, dtype=torch.int32, device=dev),
               *(torch.empty(T * k, dtype=torch.int32, device=dev) for _ in range(3)))
    offsets, row_token, row_slot, slot_row = out
    p = problem(T, 64, 64, E, k)
    if ws is None:
        ws, n = _workspace(p, CALL_DISPATCH, dev)
    else:
        n = ws.numel()
    _check("moe_dispatch", lib.moe_dispatch(_ptr(topk_idx), T, E, k, _ptr(offsets), _ptr(row_token),
                                            _ptr(row_slot), _ptr(slot_row), _ptr(ws), n, _stream()))
    return offsets, row_token, row_slot, slot_row


def pack_weights(W: torch.Tensor) -> torch.Tensor:
    """[E, K, N] bf16 -> [E, N, K] bf16 (contraction axis contiguous)."""
    _expect(W, "W", torch.bfloat16)
    E, K, N = W.shape
    Wt = torch.empty(E, N, K, dtype=torch.bfloat16, device=W.device)
    _check("moe_pack_weights", lib.moe_pack_weights(_ptr(W), E, K, N, _ptr(Wt), _stream()))
    return Wt


def mx_quantize(x: torch.Tensor):
    """bf16 [..., K] -> (E4M3 codes uint8 [..., K], E8M0 scales uint8 [..., K/32])."""
    _expect(x, "x", torch.bfloat16)
    K = x.shape[-1]
    rows = x.numel() // K
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = torch.empty(*x.shape[:-1], K // 32, dtype=torch.uint8, device=x.device)
    _check("moe_mx_quantize", lib.moe_mx_quantize(_ptr(x), rows, K, _ptr(q), _ptr(s), _stream()))
    return q, s


def expert_mlp(X, row_token, offsets, Wg_t, Wu_t, Wd_t, k, scales=None, H_rows=None, O_rows=None, ws=None,
               activation="swiglu", act_limit=0.0, static_ws=False):
    """Expert MLP over the dispatched rows.  bf16 weights [E, I, H] / [E, H, I]
    (pack_weights), or MXFP8 codes with ``scales = (Sg, Su, Sd)``.  For ReLU^2 the
    gate weight (and Sg) is None.  ``static_ws`` calls moe_expert_mlp_static (the
    library's static workspace; ``ws`` must then be None)."""
    T, H = X.shape
    E, I, _ = Wu_t.shape
    mx = scales is not None
    gated = activation not in UNGATED
    _expect(X, "X", torch.bfloat16, (T, H))
    wdt = torch.uint8 if mx else torch.bfloat16
    if gated:
        _expect(Wg_t, "Wg_t", wdt, (E, I, H))
    _expect(Wu_t, "Wu_t", wdt, (E, I, H))
    _expect(Wd_t, "Wd_t", wdt, (E, H, I))
    _expect(offsets, "expert_offsets", torch.int32, (E + 1,))
    _expect(row_token, "row_token", torch.int32, (T * k,))
    if mx:
        Sg, Su, Sd = scales
        if gated:
            _expect(Sg, "Sg", torch.uint8, (E, I, H // 32))
        _expect(Su, "Su", torch.uint8, (E, I, H // 32))
        _expect(Sd, "Sd", torch.uint8, (E, H, I // 32))
    else:
        Sg = Su = Sd = None
    dev = X.device
    H_rows = torch.empty(T * k, I, dtype=torch.bfloat16, device=dev) if H_rows is None else H_rows
    O_rows = torch.empty(T * k, H, dtype=torch.bfloat16, device=dev) if O_rows is None else O_rows
    _expect(H_rows, "H_rows", torch.bfloat16, (T * k, I))
    _expect(O_rows, "O_rows", torch.bfloat16, (T * k, H))
    p = problem(T, H, I, E, k, "mxfp8" if mx else "bf16", activation, act_limit)
    if static_ws:
        if ws is not None:
            raise ValueError("static_ws takes no workspace")
        _check("moe_expert_mlp_static",
               lib.moe_expert_mlp_static(ctypes.byref(p), _ptr(X), _ptr(row_token), _ptr(offsets), _ptr(Wg_t),
                                         _ptr(Wu_t), _ptr(Wd_t), _ptr(Sg), _ptr(Su), _ptr(Sd), _ptr(H_rows),
                                         _ptr(O_rows), _stream()))
        return H_rows, O_rows
    if ws is None:
        ws, n = _workspace(p, CALL_EXPERT_MLP, dev)
    else:
        n = ws.numel()
    _check("moe_expert_mlp", lib.moe_expert_mlp(ctypes.byref(p), _ptr(X), _ptr(row_token), _ptr(offsets),
                                                _ptr(Wg_t), _ptr(Wu_t), _ptr(Wd_t), _ptr(Sg), _ptr(Su),
                                                _ptr(Sd), _ptr(H_rows), _ptr(O_rows), _ptr(ws), n, _stream()))
    return H_rows, O_rows


def expert_mlp_save(X, row_token, offsets, Wg_t, Wu_t, Wd_t, k, H_rows=None, O_rows=None, GU_rows=None,
                    activation="swiglu", act_limit=0.0):
    """The training forward that keeps its projections (moe_expert_mlp_save, bf16): returns
    (H_rows, O_rows, GU_rows) with GU_rows [T*k, 2I] fp32, G in columns [0, I) and U in [I, 2I)."""
    T, H = X.shape
    E, I, _ = Wu_t.shape
    gated = activation not in UNGATED
    _expect(X, "X", torch.bfloat16, (T, H))
    if gated:
        _expect(Wg_t, "Wg_t", torch.bfloat16, (E, I, H))
    _expect(Wu_t, "Wu_t", torch.bfloat16, (E, I, H))
    _expect(Wd_t, "Wd_t", torch.bfloat16, (E, H, I))
    _expect(offsets, "expert_offsets", torch.int32, (E + 1,))
    _expect(row_token, "row_token", torch.int32, (T * k,))
    dev = X.device
    H_rows = torch.empty(T * k, I, dtype=torch.bfloat16, device=dev) if H_rows is None else H_rows
    O_rows = torch.empty(T * k, H, dtype=torch.bfloat16, device=dev) if O_rows is None else O_rows
    GU_rows = torch.empty(T * k, 2 * I, dtype=torch.float32, device=dev) if GU_rows is None else GU_rows
    _expect(H_rows, "H_rows", torch.bfloat16, (T * k, I))
    _expect(O_rows, "O_rows", torch.bfloat16, (T * k, H))
    _expect(GU_rows, "GU_rows", torch.float32, (T * k, 2 * I))
    p = problem(T, H, I, E, k, "bf16", activation, act_limit)
    _check("moe_expert_mlp_save", lib.moe_expert_mlp_save(ctypes.byref(p), _ptr(X), _ptr(row_token), _ptr(offsets),
                                                          _ptr(Wg_t), _ptr(Wu_t), _ptr(Wd_t), _ptr(H_rows),
                                                          _ptr(O_rows), _ptr(GU_rows), _stream()))
    return H_rows, O_rows, GU_rows


def grouped_gemm(A, B_t, m_indptr, scales=None, C=None):
    """Standalone grouped GEMM over expert-major rows: C[r] = bf16(A[r] B_t[e]^T) for the rows
    m_indptr[e] <= r < m_indptr[e+1].  bf16: A [M, K], B_t [E, N, K] (pack_weights); MXFP8:
    A and B_t as E4M3 codes with ``scales = (SA [M, K/32], SB [E, N, K/32])``."""
    M, K = A.shape
    E, N, _ = B_t.shape
    mx = scales is not None
    dt = torch.uint8 if mx else torch.bfloat16
    _expect(A, "A", dt, (M, K))
    _expect(B_t, "B_t", dt, (E, N, K))
    _expect(m_indptr, "m_indptr", torch.int32, (E + 1,))
    SA, SB = scales if mx else (None, None)
    if mx:
        _expect(SA, "SA", torch.uint8, (M, K // 32))
        _expect(SB, "SB", torch.uint8, (E, N, K // 32))
    C = torch.empty(M, N, dtype=torch.bfloat16, device=A.device) if C is None else C
    _expect(C, "C", torch.bfloat16, (M, N))
    _check("moe_grouped_gemm", lib.moe_grouped_gemm(DTYPE["mxfp8" if mx else "bf16"], _ptr(m_indptr), E, M, N, K,
                                                    _ptr(A), _ptr(SA), _ptr(B_t), _ptr(SB), _ptr(C), _stream()))
    return C


def combine(O_rows, slot_row, topk_w, Y=None):
    T, k = topk_w.shape
    H = O_rows.shape[1]
    _expect(O_rows, "O_rows", torch.bfloat16, (T * k, H))
    _expect(slot_row, "slot_row", torch.int32, (T * k,))
    _expect(topk_w, "topk_w", torch.float32, (T, k))
    Y = torch.empty(T, H, dtype=torch.bfloat16, device=O_rows.device) if Y is None else Y
    _expect(Y, "Y", torch.bfloat16, (T, H))
    _check("moe_combine", lib.moe_combine(_ptr(O_rows), _ptr(slot_row), _ptr(topk_w), T, k, H, _ptr(Y),
                                          _stream()))
    return Y


def backward(X, dY, topk_w, row_token, row_slot, slot_row, offsets, Wg_t, Wu_t, Wd_t,
             out=None, ws=None, activation="swiglu", act_limit=0.0, GU_rows=None):
    """Returns (dX, dW_gate, dW_up, dW_down, d_topk_w) from the packed weights Wg_t, Wu_t
    [E, I, H] and Wd_t [E, H, I] (pack_weights); for ReLU^2 Wg_t is None and so is dW_gate.
    With ``GU_rows`` (from expert_mlp_save) it calls moe_backward_saved: G and U are read, not
    recomputed."""
    T, H = X.shape
    E, I, _ = Wu_t.shape
    k = topk_w.shape[1]
    gated = activation not in UNGATED
    for name, t, shape in (("X", X, (T, H)), ("dY", dY, (T, H)), ("Wg_t", Wg_t, (E, I, H)),
                           ("Wu_t", Wu_t, (E, I, H)), ("Wd_t", Wd_t, (E, H, I))):
        if gated or name != "Wg_t":
            _expect(t, name, torch.bfloat16, shape)
    _expect(topk_w, "topk_w", torch.float32, (T, k))
    for name, t in (("row_token", row_token), ("row_slot", row_slot), ("slot_row", slot_row)):
        _expect(t, name, torch.int32, (T * k,))
    _expect(offsets, "expert_offsets", torch.int32, (E + 1,))
    dev = X.device
    if out is None:
        out = (torch.empty(T, H, dtype=torch.bfloat16, device=dev),
               torch.empty(E, H, I, dtype=torch.bfloat16, device=dev) if gated else None,
               torch.empty(E, H, I, dtype=torch.bfloat16, device=dev),
               torch.empty(E, I, H, dtype=torch.bfloat16, device=dev),
               torch.empty(T, k, dtype=torch.float32, device=dev))
    dX, dWg, dWu, dWd, dtw = out
    p = problem(T, H, I, E, k, "bf16", activation, act_limit)
    if ws is None:
        ws, n = _workspace(p, CALL_BACKWARD, dev)
    else:
        n = ws.numel()
    if GU_rows is not None:
        _expect(GU_rows, "GU_rows", torch.float32, (T * k, 2 * I))
        _check("moe_backward_saved",
               lib.moe_backward_saved(ctypes.byref(p), _ptr(X), _ptr(dY), _ptr(topk_w), _ptr(row_token),
                                      _ptr(row_slot), _ptr(slot_row), _ptr(offsets), _ptr(Wg_t), _ptr(Wu_t),
                                      _ptr(Wd_t), _ptr(GU_rows), _ptr(dX), _ptr(dWg), _ptr(dWu), _ptr(dWd),
                                      _ptr(dtw), _ptr(ws), n, _stream()))
        return dX, dWg, dWu, dWd, dtw
    _check("moe_backward", lib.moe_backward(ctypes.byref(p), _ptr(X), _ptr(dY), _ptr(topk_w), _ptr(row_token),
                                            _ptr(row_slot), _ptr(slot_row), _ptr(offsets), _ptr(Wg_t),
                                            _ptr(Wu_t), _ptr(Wd_t), _ptr(dX), _ptr(dWg), _ptr(dWu), _ptr(dWd),
                                            _ptr(dtw), _ptr(ws), n, _stream()))
    return dX, dWg, dWu, dWd, dtw
