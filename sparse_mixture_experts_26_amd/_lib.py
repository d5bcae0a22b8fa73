"""ctypes binding of libmoe.so: argument marshalling only.

Every function has the name and argument order of the C entry point it wraps
(include/moe.h).  Tensor arguments are torch tensors on the GPU (or None for a
NULL pointer); their ``data_ptr()`` is passed through.  ``stream`` defaults to
torch's current HIP stream.  A non-zero status raises ``MoeError``.  Nothing
here computes any step of the layer.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import (POINTER, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_size_t,
                    c_void_p)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_ACT_GELU, MOE_ACT_RELU, MOE_ACT_SWIGLU = 0, 1, 2
MOE_ROUTE_TOKEN_CHOICE, MOE_ROUTE_EXPERT_CHOICE = 0, 1
MOE_OVERFLOW_DROP, MOE_OVERFLOW_REROUTE = 0, 1
ACT_CODES = {"gelu": MOE_ACT_GELU, "relu": MOE_ACT_RELU, "swiglu": MOE_ACT_SWIGLU}
ROUTING_CODES = {"token": MOE_ROUTE_TOKEN_CHOICE, "expert": MOE_ROUTE_EXPERT_CHOICE}
OVERFLOW_CODES = {"drop": MOE_OVERFLOW_DROP, "reroute": MOE_OVERFLOW_REROUTE}
DTYPE_CODES = {"f32": MOE_F32, "bf16": MOE_BF16}


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", c_int64), ("d", c_int64), ("E", c_int64), ("k", c_int64), ("h", c_int64),
                ("n_shared", c_int64), ("capacity_factor", c_double), ("act", c_int32),
                ("dtype", c_int32), ("ffn_bias", c_int32), ("router_bias", c_int32),
                ("router_noise", c_int32), ("routing", c_int32), ("overflow", c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("w_g", "b_g", "w_noise", "w1", "w3", "w2", "b1", "b2",
                                        "ws1", "ws3", "ws2")]


class MoeAux(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("logits", "topk_idx", "topk_gate", "prob_sum", "counts",
                                        "offsets", "dest", "row_token", "stats", "scores",
                                        "slot", "diag", "final_expert", "hidden", "pre",
                                        "y_rows")]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("dx", "dw_g", "db_g", "dw_noise", "dw1", "dw3", "dw2",
                                        "db1", "db2", "dws1", "dws3", "dws2")]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (no CPU fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_mixture_experts_26_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        cfgp = POINTER(MoeConfig)
        vp, st = c_void_p, c_int
        sig = {
            "moe_status_string": (c_char_p, [c_int]),
            "moe_capacity": (c_int64, [cfgp]),
            "moe_routed_rows_bound": (c_int64, [cfgp]),
            "moe_workspace_bytes": (c_size_t, [cfgp]),
            "moe_route_launch_shape": (st, [cfgp, c_int, POINTER(c_int), POINTER(c_size_t)]),
            "moe_route": (st, [cfgp] + [vp] * 10 + [c_size_t, vp]),
            "moe_dispatch": (st, [cfgp] + [vp] * 8 + [c_size_t, vp]),
            "moe_dispatch_reroute": (st, [cfgp] + [vp] * 8 + [c_size_t, vp]),
            "moe_expert_ffn": (st, [cfgp, c_int64, vp, vp, vp, c_int64, c_int64, vp, vp, vp, vp,
                                    vp, vp, c_int, vp, c_size_t, vp]),
            "moe_expert_up": (st, [cfgp, c_int64, vp, vp, vp, c_int64, c_int64, vp, vp, vp, vp,
                                   vp, c_size_t, vp]),
            "moe_expert_down": (st, [cfgp, c_int64, vp, vp, c_int64, c_int64, vp, vp, vp, c_int,
                                     vp, c_size_t, vp]),
            "moe_combine": (st, [cfgp] + [vp] * 9),
            "moe_router_diagnostics": (st, [cfgp] + [vp] * 5 + [c_size_t, vp]),
            "moe_expert_choice": (st, [cfgp] + [vp] * 7),
            "moe_combine_expert_choice": (st, [cfgp] + [vp] * 9),
            "moe_layer_forward": (st, [cfgp, POINTER(MoeWeights), vp, vp, vp, vp,
                                       POINTER(MoeAux), vp, c_size_t, vp]),
            "moe_layer_forward_noalloc": (st, [cfgp, POINTER(MoeWeights), vp, vp, vp, vp,
                                               POINTER(MoeAux), vp]),
            "moe_backward_workspace_bytes": (c_size_t, [cfgp]),
            "moe_layer_backward": (st, [cfgp, POINTER(MoeWeights), vp, vp, vp, c_float, c_float,
                                        POINTER(MoeAux), POINTER(MoeGrads), vp, c_size_t, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


EXPORTS = ("moe_status_string", "moe_capacity", "moe_routed_rows_bound", "moe_workspace_bytes",
           "moe_route_launch_shape",
           "moe_route", "moe_dispatch", "moe_dispatch_reroute", "moe_expert_ffn", "moe_expert_up", "moe_expert_down",
           "moe_combine", "moe_router_diagnostics", "moe_expert_choice", "moe_combine_expert_choice",
           "moe_layer_forward", "moe_layer_forward_noalloc", "moe_backward_workspace_bytes",
           "moe_layer_backward")

MOE_NOALLOC_SCRATCH_BYTES = 128 << 20  # include/moe.h


def make_config(T, d, E, k, h, *, act="swiglu", dtype="bf16", capacity_factor=0.0,
                n_shared=0, ffn_bias=False, router_bias=False, router_noise=False,
                routing="token", overflow="drop") -> MoeConfig:
    return MoeConfig(T=T, d=d, E=E, k=k, h=h, n_shared=n_shared,
                     capacity_factor=float(capacity_factor),
                     act=ACT_CODES.get(act, act) if isinstance(act, str) else act,
                     dtype=DTYPE_CODES.get(dtype, dtype) if isinstance(dtype, str) else dtype,
                     ffn_bias=int(bool(ffn_bias)), router_bias=int(bool(router_bias)),
                     router_noise=int(bool(router_noise)),
                     routing=ROUTING_CODES.get(routing, routing) if isinstance(routing, str) else routing,
                     overflow=OVERFLOW_CODES.get(overflow, overflow) if isinstance(overflow, str) else overflow)


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ws(ws):
    if ws is None:
        return None, 0
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _check(name, status):
    if status != MOE_OK:
        raise MoeError(name, status)


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


moe_status_string = status_string


def moe_capacity(cfg: MoeConfig) -> int:
    return lib().moe_capacity(ctypes.byref(cfg))


def moe_routed_rows_bound(cfg: MoeConfig) -> int:
    return lib().moe_routed_rows_bound(ctypes.byref(cfg))


def moe_workspace_bytes(cfg: MoeConfig) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(cfg))


def moe_route_launch_shape(cfg: MoeConfig, device_logits: bool) -> tuple[int, int]:
    """(waves per 16-token router block, LDS bytes per block)."""
    waves, lds = c_int(0), c_size_t(0)
    _check("moe_route_launch_shape", lib().moe_route_launch_shape(
        ctypes.byref(cfg), int(bool(device_logits)), ctypes.byref(waves), ctypes.byref(lds)))
    return waves.value, lds.value


def moe_route(cfg, x, w_g, b_g, w_noise, eps, logits, topk_idx, topk_gate, prob_sum, ws,
              stream=None):
    wp, wn = _ws(ws)
    _check("moe_route", lib().moe_route(ctypes.byref(cfg), _p(x), _p(w_g), _p(b_g), _p(w_noise),
                                        _p(eps), _p(logits), _p(topk_idx), _p(topk_gate),
                                        _p(prob_sum), wp, wn, _stream(stream)))


def moe_dispatch(cfg, topk_idx, x, counts, offsets, dest, row_token, x_perm, ws, stream=None):
    wp, wn = _ws(ws)
    _check("moe_dispatch", lib().moe_dispatch(ctypes.byref(cfg), _p(topk_idx), _p(x), _p(counts),
                                              _p(offsets), _p(dest), _p(row_token), _p(x_perm),
                                              wp, wn, _stream(stream)))


def moe_dispatch_reroute(cfg, topk_idx, logits, counts, offsets, dest, row_token, final_expert, ws,
                         stream=None):
    wp, wn = _ws(ws)
    _check("moe_dispatch_reroute", lib().moe_dispatch_reroute(
        ctypes.byref(cfg), _p(topk_idx), _p(logits), _p(counts), _p(offsets), _p(dest),
        _p(row_token), _p(final_expert), wp, wn, _stream(stream)))


def moe_expert_ffn(cfg, n_groups, x_rows, row_token, offsets, rows_bound, group_bound, w1, w3, w2,
                   b1, b2, y_rows, accumulate, ws, stream=None):
    wp, wn = _ws(ws)
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        ctypes.byref(cfg), n_groups, _p(x_rows), _p(row_token), _p(offsets), rows_bound,
        group_bound, _p(w1), _p(w3), _p(w2), _p(b1), _p(b2), _p(y_rows), int(accumulate), wp, wn,
        _stream(stream)))


def moe_expert_up(cfg, n_groups, x_rows, row_token, offsets, rows_bound, group_bound, w1, w3, b1,
                  hidden, ws, stream=None):
    wp, wn = _ws(ws)
    _check("moe_expert_up", lib().moe_expert_up(
        ctypes.byref(cfg), n_groups, _p(x_rows), _p(row_token), _p(offsets), rows_bound,
        group_bound, _p(w1), _p(w3), _p(b1), _p(hidden), wp, wn, _stream(stream)))


def moe_expert_down(cfg, n_groups, hidden, offsets, rows_bound, group_bound, w2, b2, y_rows,
                    accumulate, ws, stream=None):
    wp, wn = _ws(ws)
    _check("moe_expert_down", lib().moe_expert_down(
        ctypes.byref(cfg), n_groups, _p(hidden), _p(offsets), rows_bound, group_bound, _p(w2),
        _p(b2), _p(y_rows), int(accumulate), wp, wn, _stream(stream)))


def moe_combine(cfg, y_rows, dest, topk_gate, y_shared, counts, prob_sum, y, stats, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(cfg), _p(y_rows), _p(dest),
                                            _p(topk_gate), _p(y_shared), _p(counts),
                                            _p(prob_sum), _p(y), _p(stats), _stream(stream)))


def moe_router_diagnostics(cfg, logits, counts, dest, diag, ws, stream=None):
    wp, wn = _ws(ws)
    _check("moe_router_diagnostics", lib().moe_router_diagnostics(
        ctypes.byref(cfg), _p(logits), _p(counts), _p(dest), _p(diag), wp, wn, _stream(stream)))


def moe_expert_choice(cfg, logits, scores, counts, offsets, row_token, slot, stream=None):
    _check("moe_expert_choice", lib().moe_expert_choice(
        ctypes.byref(cfg), _p(logits), _p(scores), _p(counts), _p(offsets), _p(row_token),
        _p(slot), _stream(stream)))


def moe_combine_expert_choice(cfg, y_rows, slot, scores, y_shared, counts, prob_sum, y, stats,
                              stream=None):
    _check("moe_combine_expert_choice", lib().moe_combine_expert_choice(
        ctypes.byref(cfg), _p(y_rows), _p(slot), _p(scores), _p(y_shared), _p(counts),
        _p(prob_sum), _p(y), _p(stats), _stream(stream)))


def moe_layer_forward(cfg, weights: dict, x, eps, logits_in, y, aux: dict | None, ws,
                      stream=None):
    """``weights`` and ``aux`` map MoeWeights / MoeAux field names to tensors."""
    w = MoeWeights(**{k: _p(v) for k, v in weights.items() if v is not None})
    a = MoeAux(**{k: _p(v) for k, v in (aux or {}).items() if v is not None})
    wp, wn = _ws(ws)
    _check("moe_layer_forward", lib().moe_layer_forward(
        ctypes.byref(cfg), ctypes.byref(w), _p(x), _p(eps), _p(logits_in), _p(y),
        ctypes.byref(a), wp, wn, _stream(stream)))


def moe_layer_forward_noalloc(cfg, weights: dict, x, eps, logits_in, y, aux: dict | None,
                              stream=None):
    """moe_layer_forward on the library's static scratch (no workspace)."""
    w = MoeWeights(**{k: _p(v) for k, v in weights.items() if v is not None})
    a = MoeAux(**{k: _p(v) for k, v in (aux or {}).items() if v is not None})
    _check("moe_layer_forward_noalloc", lib().moe_layer_forward_noalloc(
        ctypes.byref(cfg), ctypes.byref(w), _p(x), _p(eps), _p(logits_in), _p(y),
        ctypes.byref(a), _stream(stream)))


def moe_backward_workspace_bytes(cfg: MoeConfig) -> int:
    return lib().moe_backward_workspace_bytes(ctypes.byref(cfg))


def moe_layer_backward(cfg, weights: dict, x, eps, dy, g_aux, g_z, saved: dict, grads: dict, ws,
                       stream=None):
    """``saved`` maps MoeAux field names to the forward's tensors, ``grads``
    MoeGrads field names to output tensors."""
    w = MoeWeights(**{k: _p(v) for k, v in weights.items() if v is not None})
    a = MoeAux(**{k: _p(v) for k, v in saved.items() if v is not None})
    g = MoeGrads(**{k: _p(v) for k, v in grads.items() if v is not None})
    wp, wn = _ws(ws)
    _check("moe_layer_backward", lib().moe_layer_backward(
        ctypes.byref(cfg), ctypes.byref(w), _p(x), _p(eps), _p(dy), float(g_aux), float(g_z),
        ctypes.byref(a), ctypes.byref(g), wp, wn, _stream(stream)))
