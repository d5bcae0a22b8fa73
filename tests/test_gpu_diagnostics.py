"""GPU parity of the router z-loss and routing diagnostics against the oracle.

"Mixture-of-Experts & Sparse Model Scaling", Advanced Theory & Extensions and
Benchmark Datasets & Evaluation; "Mixture-of-experts Models", Level 3.  The
routing is replayed from the oracle's float32 logits, so counts and dest are
the oracle's exactly; z-loss and entropy (float32 per token, double sums)
must agree to 1e-5 relative, the count-based entries exactly (as float32).
"""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_26_amd as M
from sparse_mixture_experts_26_amd.layer import MoeLayer
from tests.gpu_util import banner, host, oracle_forward, require_gpu, upload, weights_of
from workloads import FULL, SMALL, make_inputs

pytestmark = pytest.mark.gpu

TC_SMALL = [n for n, c in SMALL.items() if c.routing == "token"]


def _check(cfg, want, diag):
    T, k, E = cfg.T, cfg.k, cfg.E
    C = O.capacity(cfg.capacity_factor, T, k, E) if cfg.capacity_factor > 0 else T
    C = min(C, T)
    ref = O.routing_diagnostics(want["logits"], want["counts"], want["kept"], want["dest"], C,
                                T, k, E)
    g = diag.astype(np.float64)
    for i, key in ((0, "z_loss"), (1, "entropy")):
        assert abs(g[i] - ref[key]) <= 1e-5 * max(1.0, abs(ref[key])), (key, g[i], ref[key])
    for i, key in ((2, "load_cv"), (3, "deviation"), (4, "peak_to_mean")):
        assert g[i] == pytest.approx(ref[key], rel=1e-6, abs=1e-6), key
    assert g[5] == np.float32(ref["overflow_total"])
    assert g[6] == np.float32(ref["tokens_fully_dropped"])
    assert g[7] == np.float32(ref["tokens_partly_dropped"])
    assert np.array_equal(diag[8:8 + E], ref["overflow"].astype(np.float32))
    assert np.array_equal(diag[8 + E:8 + 2 * E], ref["utilisation"].astype(np.float32))


@pytest.mark.parametrize("name", TC_SMALL)
def test_diagnostics_parity(name):
    require_gpu()
    cfg = SMALL[name]
    banner(f"diagnostics {name}")
    inp = make_inputs(cfg, 0)
    want = oracle_forward(inp)
    dev = upload(inp)
    layer = MoeLayer(cfg, weights_of(dev))
    got = layer.forward(dev["x"], dev.get("eps"), torch.from_numpy(want["logits"]).cuda())
    torch.cuda.synchronize()
    d1 = host(got["diag"]).copy()
    _check(cfg, want, d1)
    # the stage entry point on the same routing gives the same bits
    d2 = torch.empty_like(got["diag"])
    logits = torch.from_numpy(want["logits"]).cuda()
    M.moe_router_diagnostics(layer.cfg, logits, got["counts"], got["dest"], d2, layer.ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(d2), d1)


@pytest.mark.parametrize("name", ["finegrained_shared", "switch_top1"])
def test_diagnostics_full_size(name):
    """Drop-heavy full-size batches (Zipf-biased fine-grained layer, noisy
    Switch router), through the stage calls the benchmark times."""
    require_gpu()
    cfg = FULL[name]
    banner(f"diagnostics full {name}")
    inp = make_inputs(cfg, 0)
    want = oracle_forward(inp, tokens=np.array([0]))
    dev = upload(inp)
    layer = MoeLayer(cfg, weights_of(dev))
    logits = torch.from_numpy(want["logits"]).cuda()
    got = layer.staged(dev["x"], dev.get("eps"), logits_in=logits)
    d = torch.empty((8 + 2 * cfg.E,), dtype=torch.float32, device="cuda")
    M.moe_router_diagnostics(layer.cfg, logits, got["counts"], got["dest"], d, layer.ws)
    torch.cuda.synchronize()
    _check(cfg, want, host(d))
