"""Device-side driver of one MoE layer over the C ABI (marshalling only).

``MoeLayer`` owns the workspace and output buffers for a fixed shape and calls
either ``moe_layer_forward`` or the five stage entry points in order; every
step runs in the HIP kernels of libmoe.so.
"""
from __future__ import annotations

import torch

from . import _lib as L

WEIGHT_NAMES = ("w_g", "b_g", "w_noise", "w1", "w3", "w2", "b1", "b2", "ws1", "ws3", "ws2")


def config_of(spec) -> L.MoeConfig:
    """MoeConfig from any object with the layer-shape attributes (T, d, E, k, h,
    act, dtype, capacity_factor, n_shared, ffn_bias, router_bias, router_noise,
    and optionally routing: "token" or "expert")."""
    return L.make_config(spec.T, spec.d, spec.E, spec.k, spec.h, act=spec.act, dtype=spec.dtype,
                         capacity_factor=spec.capacity_factor, n_shared=spec.n_shared,
                         ffn_bias=spec.ffn_bias, router_bias=spec.router_bias != "none",
                         router_noise=spec.router_noise,
                         routing=getattr(spec, "routing", "token"),
                         overflow=getattr(spec, "overflow", "drop"))


class MoeLayer:
    def __init__(self, spec, weights: dict, device="cuda"):
        self.spec = spec
        self.cfg = config_of(spec)
        self.device = torch.device(device)
        self.w = {n: weights.get(n) for n in WEIGHT_NAMES}
        c = self.cfg
        T, E, k, d, h, S = c.T, c.E, c.k, c.d, c.h, c.n_shared
        self.capacity = L.moe_capacity(c)
        self.rows_bound = L.moe_routed_rows_bound(c)
        self.group_bound = min(T, self.capacity)
        self.ec = c.routing == L.MOE_ROUTE_EXPERT_CHOICE
        self.rr = c.overflow == L.MOE_OVERFLOW_REROUTE
        dev = self.device
        self.ws = torch.empty(max(L.moe_workspace_bytes(c), 256), dtype=torch.uint8, device=dev)
        out_dtype = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.out = {
            "y": torch.empty((T, d), dtype=out_dtype, device=dev),
            "logits": torch.empty((T, E), **f32),
            "topk_idx": torch.empty((T, k), **i32),
            "topk_gate": torch.empty((T, k), **f32),
            "prob_sum": torch.empty((E,), **f32),
            "counts": torch.empty((E,), **i32),
            "offsets": torch.empty((E + 1,), **i32),
            "dest": torch.empty((T, k), **i32),
            "row_token": torch.empty((max(T * k, self.rows_bound, 1),), **i32),
            "stats": torch.empty((2 * E + 2,), **f32),
        }
        if self.ec:
            self.out["scores"] = torch.empty((T, E), **f32)
            self.out["slot"] = torch.empty((T, E), **i32)
        else:
            self.out["diag"] = torch.empty((8 + 2 * E,), **f32)
        if self.rr:
            self.out["final_expert"] = torch.empty((T, k), **i32)
        rows = self.rows_bound + S * T
        self.hidden = torch.empty((max(rows, 1), h), dtype=out_dtype, device=dev)
        self.y_rows = torch.empty((max(rows, 1), d), **f32)

    def forward(self, x, eps=None, logits_in=None, stream=None, diag=True):
        """moe_layer_forward with every auxiliary output captured (the routing
        diagnostics only when ``diag``)."""
        aux = {n: self.out[n] for n in ("logits", "topk_idx", "topk_gate", "prob_sum", "counts",
                                        "offsets", "dest", "row_token", "stats", "scores", "slot",
                                        "diag", "final_expert")
               if n in self.out and (diag or n != "diag")}
        if logits_in is not None:
            aux.pop("logits")
        L.moe_layer_forward(self.cfg, self.w, x, eps, logits_in, self.out["y"], aux, self.ws,
                            stream)
        return self.out

    def staged(self, x, eps=None, logits_in=None, stream=None, between=None, scores_in=None):
        """The same layer through the five stage entry points; ``between(name)``
        is called after each stage is enqueued (for event timing).  With
        expert-choice routing, ``scores_in`` replays float32 scores [T,E]."""
        c, o, w = self.cfg, self.out, self.w
        T, d, S = c.T, c.d, c.n_shared
        tick = between or (lambda name: None)
        if logits_in is not None:
            o["logits"].copy_(logits_in)
            L.moe_route(c, None, None, None, None, None, o["logits"], o["topk_idx"],
                        o["topk_gate"], o["prob_sum"], self.ws, stream)
        else:
            L.moe_route(c, x, w["w_g"], w["b_g"], w["w_noise"], eps, o["logits"], o["topk_idx"],
                        o["topk_gate"], o["prob_sum"], self.ws, stream)
        tick("route")
        if self.ec:
            if scores_in is not None:
                o["scores"].copy_(scores_in)
            L.moe_expert_choice(c, None if scores_in is not None else o["logits"], o["scores"],
                                o["counts"], o["offsets"], o["row_token"], o["slot"], stream)
        elif self.rr:
            L.moe_dispatch_reroute(c, o["topk_idx"], o["logits"], o["counts"], o["offsets"],
                                   o["dest"], o["row_token"], o["final_expert"], self.ws, stream)
        else:
            L.moe_dispatch(c, o["topk_idx"], None, o["counts"], o["offsets"], o["dest"],
                           o["row_token"], None, self.ws, stream)
        tick("dispatch")
        R = self.rows_bound
        L.moe_expert_up(c, c.E, x, o["row_token"], o["offsets"], R, self.group_bound, w["w1"],
                        w["w3"], w["b1"], self.hidden, self.ws, stream)
        tick("up")
        L.moe_expert_down(c, c.E, self.hidden, o["offsets"], R, self.group_bound, w["w2"],
                          w["b2"], self.y_rows, 0, self.ws, stream)
        tick("down")
        y_shared = None
        if S:
            y_shared = self.y_rows[R:R + S * T]
            for s in range(S):
                off = self._shared_offsets()
                L.moe_expert_up(c, 1, x, None, off, T, T, w["ws1"][s], w["ws3"][s], None,
                                self.hidden[R:], self.ws, stream)
                L.moe_expert_down(c, 1, self.hidden[R:], off, T, T, w["ws2"][s], None,
                                  y_shared[s * T:(s + 1) * T], 0, self.ws, stream)
            tick("shared")
        if self.ec:
            L.moe_combine_expert_choice(c, self.y_rows, o["slot"], o["scores"], y_shared,
                                        o["counts"], o["prob_sum"], o["y"], o["stats"], stream)
        else:
            L.moe_combine(c, self.y_rows, o["dest"], o["topk_gate"], y_shared, o["counts"],
                          o["prob_sum"], o["y"], o["stats"], stream)
        tick("combine")
        return o

    # ---- training ------------------------------------------------------------------
    def forward_train(self, x, eps=None, logits_in=None, stream=None):
        """moe_layer_forward that also keeps what moe_layer_backward needs (the
        pre-activations, hidden layer and expert rows) in this object."""
        c = self.cfg
        if not hasattr(self, "pre"):
            rows = self.rows_bound + c.n_shared * c.T
            width = (2 if c.act == L.MOE_ACT_SWIGLU else 1) * c.h
            self.pre = torch.empty((max(rows, 1), width), dtype=self.hidden.dtype,
                                   device=self.device)
        aux = {n: self.out[n] for n in ("logits", "topk_idx", "topk_gate", "prob_sum", "counts",
                                        "offsets", "dest", "row_token", "stats", "scores", "slot",
                                        "diag", "final_expert")
               if n in self.out}
        aux.update(hidden=self.hidden, pre=self.pre, y_rows=self.y_rows)
        if logits_in is not None:
            aux.pop("logits")
        L.moe_layer_forward(c, self.w, x, eps, logits_in, self.out["y"], aux, self.ws, stream)
        self._saved = dict(aux, logits=logits_in if logits_in is not None else self.out["logits"])
        return self.out

    def backward(self, x, dy, eps=None, g_aux=0.0, g_z=0.0, stream=None) -> dict:
        """moe_layer_backward after ``forward_train`` on the same batch: float32
        gradients of <dy, y> + g_aux L_aux + g_z L_z."""
        c = self.cfg
        T, d, E, h, S = c.T, c.d, c.E, c.h, c.n_shared
        dev = self.device
        if not hasattr(self, "grads"):
            f32 = dict(dtype=torch.float32, device=dev)
            swi = c.act == L.MOE_ACT_SWIGLU
            g = {"dx": torch.empty((T, d), **f32), "dw_g": torch.empty((E, d), **f32),
                 "dw1": torch.empty((E, h, d), **f32), "dw2": torch.empty((E, d, h), **f32)}
            if swi:
                g["dw3"] = torch.empty((E, h, d), **f32)
            if c.router_bias:
                g["db_g"] = torch.empty((E,), **f32)
            if c.router_noise:
                g["dw_noise"] = torch.empty((E, d), **f32)
            if c.ffn_bias:
                g["db1"] = torch.empty((E, h), **f32)
                g["db2"] = torch.empty((E, d), **f32)
            if S:
                g["dws1"] = torch.empty((S, h, d), **f32)
                g["dws2"] = torch.empty((S, d, h), **f32)
                if swi:
                    g["dws3"] = torch.empty((S, h, d), **f32)
            self.grads = g
            self.bws = torch.empty(max(L.moe_backward_workspace_bytes(c), 256), dtype=torch.uint8,
                                   device=dev)
        L.moe_layer_backward(c, self.w, x, eps, dy, g_aux, g_z, self._saved, self.grads, self.bws,
                             stream)
        return self.grads

    def _shared_offsets(self):
        if not hasattr(self, "_soff"):
            self._soff = torch.tensor([0, self.cfg.T], dtype=torch.int32, device=self.device)
        return self._soff
