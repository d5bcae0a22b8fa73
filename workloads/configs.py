"""Layer shapes of the five sparse-MoE workloads, plus reduced variants for tests.

Shapes and distributions follow the workload descriptions that accompany the
pages (a toy fp32 layer, a Switch-style top-1 layer, a Mixtral-shaped decode
batch and prefill, and a fine-grained layer with shared experts).  This module
holds shapes only; no step of the layer is computed here.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

ACTS = ("gelu", "relu", "swiglu")
DTYPES = ("f32", "bf16")


@dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int          # seeds the input streams; reduced variants get their own id
    T: int               # tokens in the batch
    d: int               # model width
    E: int               # routed experts
    k: int               # experts per token
    h: int               # expert hidden width
    act: str             # "gelu" | "relu" | "swiglu"
    capacity_factor: float  # <= 0 means dropless
    dtype: str           # "f32" | "bf16": activations and weights
    n_shared: int = 0    # always-on shared experts (same act and h as the routed ones)
    ffn_bias: bool = False
    router_noise: bool = False
    router_bias: str = "none"   # "none" | "normal" | "zipf"
    router_bias_std: float = 0.0
    zipf_s: float = 0.0
    x_std: float = 1.0
    w_std: float = 0.02
    b_std: float = 0.02          # std of b1/b2 where ffn_bias is set
    routing: str = "token"       # "token": top-k per token; "expert": top-C' per expert
    overflow: str = "drop"       # "drop" | "reroute": what a full expert does to an assignment

    @property
    def dropless(self) -> bool:
        return self.capacity_factor <= 0.0

    @property
    def gated(self) -> bool:
        return self.act == "swiglu"

    def with_(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


TOY = LayerConfig(
    name="toy_fp32", cfg_id=1, T=64, d=64, E=4, k=2, h=128, act="gelu",
    capacity_factor=1.25, dtype="f32", ffn_bias=True)

SWITCH = LayerConfig(
    name="switch_top1", cfg_id=2, T=4096, d=768, E=128, k=1, h=3072, act="relu",
    capacity_factor=1.0, dtype="bf16", router_noise=True)

DECODE = LayerConfig(
    name="mixtral_decode", cfg_id=3, T=32, d=4096, E=8, k=2, h=14336, act="swiglu",
    capacity_factor=0.0, dtype="bf16")

PREFILL = LayerConfig(
    name="mixtral_prefill", cfg_id=4, T=8192, d=4096, E=8, k=2, h=14336, act="swiglu",
    capacity_factor=0.0, dtype="bf16", router_bias="normal", router_bias_std=0.5)

FINEGRAINED = LayerConfig(
    name="finegrained_shared", cfg_id=5, T=16384, d=2048, E=64, k=6, h=1408, act="swiglu",
    capacity_factor=1.25, dtype="bf16", n_shared=2, router_bias="zipf", zipf_s=1.1)

# Expert-choice routing on the Mixtral prefill shape: capacity factor 1.0
# gives every expert C = T*k/E = 2048 tokens (the same rows as top-2 on
# average, now perfectly balanced).
PREFILL_EC = PREFILL.with_(name="mixtral_prefill_ec", cfg_id=6, capacity_factor=1.0,
                           routing="expert")

# The fine-grained layer again, with overflow re-routed to lower-ranked
# experts instead of dropped (its Zipf-biased router overflows 62% of the
# assignments when they are dropped).
FINEGRAINED_RR = FINEGRAINED.with_(name="finegrained_reroute", cfg_id=7, overflow="reroute")

FULL = {c.name: c for c in (TOY, SWITCH, DECODE, PREFILL, FINEGRAINED, PREFILL_EC,
                            FINEGRAINED_RR)}

# Reduced variants: same structure (act, k, noise, bias kind, shared experts,
# capacity regime), sizes small enough for the CPU oracle to finish in seconds,
# chosen so that every GEMM spans several tiles and ends in a ragged tail.
SMALL = {
    "toy_fp32": TOY,
    "switch_small": SWITCH.with_(name="switch_small", cfg_id=102, T=1000, d=256, E=16,
                                 h=384),
    "decode_small": DECODE.with_(name="decode_small", cfg_id=103, T=21, d=512, E=8,
                                 h=1216),
    "prefill_small": PREFILL.with_(name="prefill_small", cfg_id=104, T=777, d=384, E=8,
                                   h=704),
    "finegrained_small": FINEGRAINED.with_(name="finegrained_small", cfg_id=105, T=1500,
                                           d=256, E=16, k=4, h=192, n_shared=2),
    "prefill_ec_small": PREFILL_EC.with_(name="prefill_ec_small", cfg_id=106, T=777, d=384,
                                         E=8, h=704),
    "finegrained_ec_small": FINEGRAINED.with_(name="finegrained_ec_small", cfg_id=107, T=1500,
                                              d=256, E=16, k=4, h=192, n_shared=2,
                                              routing="expert"),
    "finegrained_rr_small": FINEGRAINED_RR.with_(name="finegrained_rr_small", cfg_id=108,
                                                 T=1500, d=256, E=16, k=4, h=192, n_shared=2),
    "switch_rr_small": SWITCH.with_(name="switch_rr_small", cfg_id=109, T=1000, d=256, E=16,
                                    h=384, overflow="reroute"),
}


def capacity_note(cfg: LayerConfig) -> str:
    return "dropless" if cfg.dropless else f"capacity factor {cfg.capacity_factor}"
