"""Seeded synthetic workloads (shapes and input tensors) for the sparse-MoE layer.

Serves both the CPU oracle and the HIP path with identical inputs; it holds no
step of the layer itself.
"""
from .configs import FULL, SMALL, LayerConfig, TOY, SWITCH, DECODE, PREFILL, FINEGRAINED
from .generate import (LayerInputs, make_inputs, make_upstream_grad, round_to_bf16_bits,
                       router_bias, to_torch)
