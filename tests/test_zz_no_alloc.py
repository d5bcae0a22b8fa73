"""moe_layer_forward_noalloc (the layer on the library's static scratch, for
callers that cannot allocate) against moe_layer_forward on a caller-owned
workspace, through the C ABI.  Both run the same kernels in the same order,
so every output must be bit-identical.  Two calls in a row on one device
share the scratch; the second is a smaller layer of another shape, so
whatever the first left behind must not leak into it.  The first call of the
process also performs the one-time lookup of the scratch's device address.
"""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_26_amd as M
from sparse_mixture_experts_26_amd.layer import MoeLayer
from tests.gpu_util import banner, oracle_forward, rel_l2, require_gpu, upload, weights_of
from workloads import SMALL, make_inputs

pytestmark = pytest.mark.gpu

AUX = ("logits", "topk_idx", "topk_gate", "prob_sum", "counts", "offsets", "dest", "row_token",
       "stats", "diag")


def _outputs(layer, fill):
    o = {n: torch.empty_like(layer.out[n]) for n in AUX}
    o["y"] = torch.empty_like(layer.out["y"])
    for t in o.values():
        t.fill_(fill) if t.dtype == torch.int32 else t.fill_(float(fill))
    return o


def _bits(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    elif t.dtype == torch.float32:
        t = t.view(torch.int32)
    return t.cpu().numpy()


def _run_pair(name):
    cfg = SMALL[name]
    banner(f"noalloc {name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} h={cfg.h} S={cfg.n_shared}")
    inp = make_inputs(cfg, seed=1)
    dev = upload(inp)
    layer = MoeLayer(cfg, weights_of(dev))
    x, eps = dev["x"], dev.get("eps")
    # the existing entry point, on the layer's own workspace
    ref = _outputs(layer, -5)
    M.moe_layer_forward(layer.cfg, layer.w, x, eps, None, ref["y"],
                        {n: ref[n] for n in AUX}, layer.ws)
    # the scratch variant, outputs poisoned differently
    got = _outputs(layer, -9)
    M.moe_layer_forward_noalloc(layer.cfg, layer.w, x, eps, None, got["y"],
                                {n: got[n] for n in AUX})
    torch.cuda.synchronize()
    total = int(ref["offsets"][-1].item())
    for n in ("y",) + AUX:
        a, b = _bits(ref[n]), _bits(got[n])
        if n == "row_token":
            a, b = a[:total], b[:total]
        assert np.array_equal(a, b), (name, n)
    # and both are the layer the oracle computes on these logits
    want = oracle_forward(inp, logits=ref["logits"].cpu().numpy())
    assert np.array_equal(ref["dest"].cpu().numpy(), want["dest"])
    y = got["y"].float().cpu().numpy()
    assert rel_l2(y, want["y"]) <= 2e-2
    return cfg


def test_noalloc_matches_workspace_call_twice_shrinking():
    require_gpu()
    big = _run_pair("finegrained_small")   # 18.8 MiB of scratch, shared experts, drops
    small = _run_pair("decode_small")      # 2.4 MiB, the weight-streaming kernels
    assert small.T < big.T


def test_noalloc_noisy_after_larger():
    require_gpu()
    _run_pair("switch_small")              # noisy router, capacity drops
    _run_pair("toy_fp32")                  # float32 end to end, smaller again
