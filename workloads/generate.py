"""Seeded synthetic inputs for the sparse-MoE workloads.

Every tensor comes from its own counter-free numpy stream,
``np.random.default_rng(SeedSequence([seed, cfg_id, tensor_id, sub]))``, where
``sub`` is the expert index for per-expert weights (so one expert's weights can
be regenerated alone) and 0 otherwise.  Draws are float32 standard normals
scaled by the configured std; bf16 workloads then round to bfloat16 with
round-to-nearest-even and keep the raw 16-bit patterns (``np.uint16``).

Recipe per tensor (std values come from the config):
  x        [T, d]      N(0, x_std^2)
  w_g      [E, d]      N(0, w_std^2)
  b_g      [E]  fp32   "normal": N(0, router_bias_std^2); "zipf": -s*ln(e+1), so
                       that softmax(b_g) is the Zipf(s) pmf over expert ranks
  w_noise  [E, d]      N(0, w_std^2)                        (noisy gating only)
  eps      [T, E] fp32 N(0, 1)                              (noisy gating only)
  w1, w3   [E, h, d]   N(0, w_std^2)   (w3 only for the gated activation)
  w2       [E, d, h]   N(0, w_std^2)
  b1 [E, h], b2 [E, d] fp32 N(0, b_std^2)                   (ffn_bias only)
  ws1, ws3 [S, h, d], ws2 [S, d, h]   shared experts, N(0, w_std^2)
  dy       [T, d] fp32 N(0, 1)   upstream gradient of the layer output (backward)

No step of the layer is computed here.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .configs import LayerConfig

TENSOR_IDS = {
    "x": 0, "w_g": 1, "b_g": 2, "w_noise": 3, "eps": 4,
    "w1": 5, "w3": 6, "w2": 7, "b1": 8, "b2": 9,
    "ws1": 10, "ws3": 11, "ws2": 12, "dy": 13,
}


def _rng(seed: int, cfg_id: int, name: str, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg_id, TENSOR_IDS[name], sub]))


def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16_bits(a) if dtype == "bf16" else a.astype(np.float32, copy=False)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@dataclass
class LayerInputs:
    cfg: LayerConfig
    seed: int
    x: np.ndarray
    w_g: np.ndarray
    w1: np.ndarray
    w2: np.ndarray
    w3: np.ndarray | None = None
    b_g: np.ndarray | None = None
    w_noise: np.ndarray | None = None
    eps: np.ndarray | None = None
    b1: np.ndarray | None = None
    b2: np.ndarray | None = None
    ws1: np.ndarray | None = None
    ws3: np.ndarray | None = None
    ws2: np.ndarray | None = None
    extra: dict = field(default_factory=dict)

    def tensors(self) -> dict:
        names = ("x", "w_g", "b_g", "w_noise", "eps", "w1", "w3", "w2", "b1", "b2",
                 "ws1", "ws3", "ws2")
        return {n: getattr(self, n) for n in names if getattr(self, n) is not None}


def _per_expert(seed, cfg, name, n, shape, std, dtype) -> np.ndarray:
    """Stack of n slabs, slab e drawn from stream (seed, cfg_id, name, e)."""
    out = np.empty((n,) + tuple(shape), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def one(e):
        out[e] = _store(_normal(_rng(seed, cfg.cfg_id, name, e), shape, std), dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(n)))
    return out


def router_bias(cfg: LayerConfig, seed: int = 0) -> np.ndarray | None:
    if cfg.router_bias == "none":
        return None
    if cfg.router_bias == "normal":
        return _normal(_rng(seed, cfg.cfg_id, "b_g"), (cfg.E,), cfg.router_bias_std)
    if cfg.router_bias == "zipf":
        ranks = np.arange(1, cfg.E + 1, dtype=np.float64)
        return (-cfg.zipf_s * np.log(ranks)).astype(np.float32)
    raise ValueError(cfg.router_bias)


def make_inputs(cfg: LayerConfig, seed: int = 0, experts: bool = True) -> LayerInputs:
    """All inputs of one layer.  ``experts=False`` skips the expert weights."""
    T, d, E, h, S = cfg.T, cfg.d, cfg.E, cfg.h, cfg.n_shared
    dt = cfg.dtype
    x = _store(_normal(_rng(seed, cfg.cfg_id, "x"), (T, d), cfg.x_std), dt)
    w_g = _store(_normal(_rng(seed, cfg.cfg_id, "w_g"), (E, d), cfg.w_std), dt)
    inp = LayerInputs(cfg=cfg, seed=seed, x=x, w_g=w_g,
                      w1=np.empty(0), w2=np.empty(0))
    inp.b_g = router_bias(cfg, seed)
    if cfg.router_noise:
        inp.w_noise = _store(_normal(_rng(seed, cfg.cfg_id, "w_noise"), (E, d), cfg.w_std), dt)
        inp.eps = _normal(_rng(seed, cfg.cfg_id, "eps"), (T, E), 1.0)
    if not experts:
        return inp
    inp.w1 = _per_expert(seed, cfg, "w1", E, (h, d), cfg.w_std, dt)
    inp.w2 = _per_expert(seed, cfg, "w2", E, (d, h), cfg.w_std, dt)
    if cfg.gated:
        inp.w3 = _per_expert(seed, cfg, "w3", E, (h, d), cfg.w_std, dt)
    if cfg.ffn_bias:
        inp.b1 = _per_expert(seed, cfg, "b1", E, (h,), cfg.b_std, "f32")
        inp.b2 = _per_expert(seed, cfg, "b2", E, (d,), cfg.b_std, "f32")
    if S:
        inp.ws1 = _per_expert(seed, cfg, "ws1", S, (h, d), cfg.w_std, dt)
        inp.ws2 = _per_expert(seed, cfg, "ws2", S, (d, h), cfg.w_std, dt)
        if cfg.gated:
            inp.ws3 = _per_expert(seed, cfg, "ws3", S, (h, d), cfg.w_std, dt)
    return inp


def to_torch(a: np.ndarray, device="cpu"):
    """Host array -> torch tensor; uint16 arrays become bfloat16 tensors."""
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device) if str(device) != "cpu" else t


def make_upstream_grad(cfg: LayerConfig, seed: int = 0) -> np.ndarray:
    """dy [T, d] float32 ~ N(0, 1): the gradient a training step hands the
    layer output (the backward's input)."""
    return _normal(_rng(seed, cfg.cfg_id, "dy"), (cfg.T, cfg.d), 1.0)
