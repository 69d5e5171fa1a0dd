"""Routed MoE expert layer on top of the C ABI.

``MoELayer`` owns the packed (and, for MXFP8, quantised) expert weights and,
per token count, every intermediate buffer and workspace, so that a warmed
forward or backward enqueues kernels only (no allocation) and can be captured
in a HIP graph.  The five calls run in the order the LightMoE README lists
for one inference call (dispatch, gate/up projection, gated activation, down
projection, routing-weight application and combine), preceded by routing.
"""
from __future__ import annotations

import torch

from . import binding as B


class MoELayer:
    def __init__(self, H: int, I: int, E: int, k: int, dtype: str = "bf16", device="cuda",
                 activation: str = "swiglu", act_limit: float = 0.0, save_activations: bool = False):
        """``activation``: swiglu (default), swiglu_clamp, swiglu_oai, geglu, reglu or relu2
        (include/moe.h, moe_activation; relu2 experts have no gate weight); ``act_limit``: the
        clamp of the two clamped ones.  ``save_activations`` (bf16): a forward with a backward
        plan keeps the fp32 projections G, U of every routed row (moe_expert_mlp_save) and the
        backward reads them instead of recomputing them (moe_backward_saved)."""
        if save_activations and dtype != "bf16":
            raise ValueError("saved activations are a bf16 training path")
        self.H, self.I, self.E, self.k, self.dtype = H, I, E, k, dtype
        self.activation, self.act_limit = activation, act_limit
        self.save_activations = save_activations
        self.device = torch.device(device)
        self._plans = {}

    # -- weights (once, outside any timed region) ---------------------------------
    def load_weights(self, W_gate, W_up: torch.Tensor, W_down: torch.Tensor):
        """W_gate, W_up [E, H, I] and W_down [E, I, H] bf16 on the device (W_gate None for the
        two-weight ReLU^2 expert).  The layer keeps only the packed copies (forward and backward
        both read them; the caller's tensors may be freed)."""
        if (W_gate is None) != (self.activation in B.UNGATED):
            raise ValueError("ReLU^2 experts take no gate weight; every other activation needs one")
        self.Wg_t = B.pack_weights(W_gate) if W_gate is not None else None
        self.Wu_t = B.pack_weights(W_up)
        self.Wd_t = B.pack_weights(W_down)
        self.scales = None
        if self.dtype == "mxfp8":
            qg, sg = B.mx_quantize(self.Wg_t) if self.Wg_t is not None else (None, None)
            qu, su = B.mx_quantize(self.Wu_t)
            qd, sd = B.mx_quantize(self.Wd_t)
            self.Wg_t, self.Wu_t, self.Wd_t = qg, qu, qd
            self.scales = (sg, su, sd)
        return self

    # -- buffers per token count ------------------------------------------------------
    def plan(self, T: int, backward: bool = False):
        key = (T, backward)
        if key in self._plans:
            return self._plans[key]
        H, I, E, k, dev = self.H, self.I, self.E, self.k, self.device
        A = T * k
        p = B.problem(T, H, I, E, k, self.dtype, self.activation, self.act_limit)
        pl = {
            "topk_idx": torch.empty(T, k, dtype=torch.int32, device=dev),
            "topk_w": torch.empty(T, k, dtype=torch.float32, device=dev),
            "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "row_token": torch.empty(A, dtype=torch.int32, device=dev),
            "row_slot": torch.empty(A, dtype=torch.int32, device=dev),
            "slot_row": torch.empty(A, dtype=torch.int32, device=dev),
            "H_rows": torch.empty(A, I, dtype=torch.bfloat16, device=dev),
            "O_rows": torch.empty(A, H, dtype=torch.bfloat16, device=dev),
            "Y": torch.empty(T, H, dtype=torch.bfloat16, device=dev),
            "ws_dispatch": torch.empty(max(1, B.workspace_size(p, B.CALL_DISPATCH)), dtype=torch.uint8, device=dev),
            "ws_mlp": torch.empty(max(1, B.workspace_size(p, B.CALL_EXPERT_MLP)), dtype=torch.uint8, device=dev),
        }
        if backward:
            pl["ws_bwd"] = torch.empty(B.workspace_size(p, B.CALL_BACKWARD), dtype=torch.uint8, device=dev)
            if self.save_activations:
                pl["GU"] = torch.empty(A, 2 * I, dtype=torch.float32, device=dev)
            pl["grads"] = (torch.empty(T, H, dtype=torch.bfloat16, device=dev),
                           torch.empty(E, H, I, dtype=torch.bfloat16, device=dev)
                           if self.activation not in B.UNGATED else None,
                           torch.empty(E, H, I, dtype=torch.bfloat16, device=dev),
                           torch.empty(E, I, H, dtype=torch.bfloat16, device=dev),
                           torch.empty(T, k, dtype=torch.float32, device=dev))
        self._plans[key] = pl
        return pl

    # -- forward / backward -----------------------------------------------------------
    def forward(self, logits: torch.Tensor, X: torch.Tensor, backward_plan: bool = False, mlp_events=None):
        """Runs route, dispatch, expert MLP and combine on the current stream.
        ``mlp_events`` = (start, end) timing events (objects with ``record()``, such as
        torch.cuda.Event) recorded around the expert MLP call on the current stream,
        the stream of its kernels."""
        T = X.shape[0]
        pl = self.plan(T, backward_plan)
        B.route(logits, self.k, pl["topk_idx"], pl["topk_w"])
        B.dispatch(pl["topk_idx"], self.E, (pl["offsets"], pl["row_token"], pl["row_slot"], pl["slot_row"]),
                   ws=pl["ws_dispatch"])
        if mlp_events is not None:
            mlp_events[0].record()
        self._expert_mlp(X, pl)
        if mlp_events is not None:
            mlp_events[1].record()
        B.combine(pl["O_rows"], pl["slot_row"], pl["topk_w"], pl["Y"])
        return pl["Y"]

    def _expert_mlp(self, X: torch.Tensor, pl):
        if "GU" in pl:
            B.expert_mlp_save(X, pl["row_token"], pl["offsets"], self.Wg_t, self.Wu_t, self.Wd_t, self.k,
                              H_rows=pl["H_rows"], O_rows=pl["O_rows"], GU_rows=pl["GU"],
                              activation=self.activation, act_limit=self.act_limit)
        else:
            B.expert_mlp(X, pl["row_token"], pl["offsets"], self.Wg_t, self.Wu_t, self.Wd_t, self.k,
                         scales=self.scales, H_rows=pl["H_rows"], O_rows=pl["O_rows"], ws=pl["ws_mlp"],
                         activation=self.activation, act_limit=self.act_limit)

    def forward_routed(self, topk_idx: torch.Tensor, topk_w: torch.Tensor, X: torch.Tensor,
                       backward_plan: bool = False):
        """The layer with the routing given by the caller (LightMoE "MoE inference": the call takes
        the top-k ids, int32 with distinct experts per token, and their fp32 weights): dispatch,
        expert MLP and combine.  The ids and weights are copied into the plan, so that a following
        ``backward`` sees them.  An id outside [0, E) is skipped as moe_dispatch documents: its slot
        adds nothing to Y (and gets d_topk_w = 0)."""
        T = X.shape[0]
        pl = self.plan(T, backward_plan)
        for name, t, dt in (("topk_idx", topk_idx, torch.int32), ("topk_w", topk_w, torch.float32)):
            if t.dtype != dt or tuple(t.shape) != (T, self.k) or t.device.type != self.device.type:
                raise ValueError(f"{name} must be a [{T}, {self.k}] {dt} tensor on {self.device}")
        pl["topk_idx"].copy_(topk_idx)
        pl["topk_w"].copy_(topk_w)
        B.dispatch(pl["topk_idx"], self.E, (pl["offsets"], pl["row_token"], pl["row_slot"], pl["slot_row"]),
                   ws=pl["ws_dispatch"])
        self._expert_mlp(X, pl)
        B.combine(pl["O_rows"], pl["slot_row"], pl["topk_w"], pl["Y"])
        return pl["Y"]

    def run_routed(self, x_rows: torch.Tensor, m_indptr: torch.Tensor):
        """The expert MLP over rows already in expert-major order (LightMoE "MoE inference":
        frameworks with expert-major input): O[r] = MLP_e(x_rows[r]) for the rows
        m_indptr[e] <= r < m_indptr[e+1] of every expert; no routing weights, no combine.
        Returns O [rows, H] bf16."""
        A = x_rows.shape[0]
        key = ("rows", A)
        if key not in self._plans:
            self._plans[key] = torch.arange(A, dtype=torch.int32, device=self.device)
        _, O = B.expert_mlp(x_rows, self._plans[key], m_indptr, self.Wg_t, self.Wu_t, self.Wd_t, 1,
                            scales=self.scales, activation=self.activation, act_limit=self.act_limit)
        return O

    def backward(self, X: torch.Tensor, dY: torch.Tensor):
        """Gradients of the last forward with the same X (needs backward_plan=True)."""
        if self.dtype != "bf16":
            raise ValueError("the backward runs on bf16 weights")
        T = X.shape[0]
        pl = self.plan(T, True)
        return B.backward(X, dY, pl["topk_w"], pl["row_token"], pl["row_slot"], pl["slot_row"], pl["offsets"],
                          self.Wg_t, self.Wu_t, self.Wd_t, out=pl["grads"],
                          ws=pl["ws_bwd"], activation=self.activation, act_limit=self.act_limit,
                          GU_rows=pl.get("GU"))

    def route_backward(self, T: int):
        """Gradient with respect to the router logits [T, E] fp32, from the d(top-k weights) of the
        last backward over T tokens."""
        pl = self.plan(T, True)
        if "d_logits" not in pl:
            pl["d_logits"] = torch.empty(T, self.E, dtype=torch.float32, device=self.device)
        return B.route_backward(pl["topk_idx"], pl["topk_w"], pl["grads"][4], self.E, pl["d_logits"])
