"""Helpers shared by the GPU parity tests: device upload, oracle calls, metrics."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from workloads import to_torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_mixture_experts_26_amd as M
    M.lib()  # a missing build fails here, loudly


def upload(inp, device="cuda") -> dict:
    return {k: to_torch(v, device) for k, v in inp.tensors().items()}


def oracle_forward(inp, logits=None, tokens=None) -> dict:
    c = inp.cfg
    return O.moe_forward(inp.x, inp.w_g, inp.w1, inp.w2, k=c.k, act=c.act,
                         capacity_factor=c.capacity_factor, w3=inp.w3, b_g=inp.b_g,
                         w_noise=inp.w_noise, eps=inp.eps, b1=inp.b1, b2=inp.b2,
                         ws1=inp.ws1, ws3=inp.ws3, ws2=inp.ws2, logits=logits, tokens=tokens,
                         overflow=c.overflow)


def weights_of(dev: dict) -> dict:
    return {n: dev.get(n) for n in ("w_g", "b_g", "w_noise", "w1", "w3", "w2", "b1", "b2",
                                    "ws1", "ws3", "ws2")}


def host(t) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def rel_l2(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def y_tol(cfg) -> float:
    """Output tolerance: 2e-2 relative L2 for bf16 layers, 1e-5 for float32."""
    return 2e-2 if cfg.dtype == "bf16" else 1e-5


def banner(msg: str):
    print(f"[gpu-case] {msg}", flush=True)


def row_tol(cfg) -> float:
    """Per-token output tolerance (relative L2 of one row): 5e-2 for bf16
    layers, 1e-5 for float32.  A whole-tensor relative L2 over thousands of
    tokens would let one wholly wrong token through."""
    return 5e-2 if cfg.dtype == "bf16" else 1e-5


def worst_row_error(got, want) -> float:
    """Largest per-row relative L2 error; a row whose reference is exactly
    zero (a token with every assignment dropped and no shared expert) must be
    exactly zero too (reported as inf otherwise)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    num = np.linalg.norm(got - want, axis=1)
    den = np.linalg.norm(want, axis=1)
    zero = den == 0
    if np.any(num[zero] != 0):
        return float("inf")
    return float(np.max(num[~zero] / den[~zero], initial=0.0))


def topk_flips(H_ref, H_gpu, k):
    """Tokens whose top-k expert set differs between the two float32 logit
    matrices, and each such token's gap between its k-th and (k+1)-th
    reference logits (0 when k = E)."""
    a = np.sort(O.select_top_k(np.asarray(H_ref, np.float32), k), axis=1)
    b = np.sort(O.select_top_k(np.asarray(H_gpu, np.float32), k), axis=1)
    diff = np.nonzero(np.any(a != b, axis=1))[0]
    E = np.asarray(H_ref).shape[1]
    if k >= E:
        return diff, np.zeros(diff.size)
    srt = -np.sort(-np.asarray(H_ref, np.float64), axis=1)
    gap = srt[:, k - 1] - srt[:, k]
    return diff, gap[diff]
