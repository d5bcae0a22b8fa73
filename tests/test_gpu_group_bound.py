"""The group_bound contract of the stage expert FFN calls.

group_bound selects the kernel: at most 32 rows per group streams the weights
(the decode/Switch-shaped kernel), anything larger takes the tiled kernel.  A
group above 32 rows is computed correctly when group_bound says so, and when
group_bound understates it (a broken promise the host cannot see, since the
offsets live on the device) that group's output rows come back as NaN while
every other group is still computed correctly.
"""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_26_amd as M
from sparse_mixture_experts_26_amd import _lib as L
from sparse_mixture_experts_26_amd.layer import config_of
from tests.gpu_util import banner, host, rel_l2, require_gpu, worst_row_error
from workloads import LayerConfig, make_inputs, to_torch

pytestmark = pytest.mark.gpu


def _setup(sizes, act="swiglu"):
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offsets[-1])
    cfg = LayerConfig(name="group_bound", cfg_id=72, T=96, d=256, E=G, k=1, h=192, act=act,
                      capacity_factor=0.0, dtype="bf16")
    inp = make_inputs(cfg, seed=5)
    row_token = ((np.arange(rows, dtype=np.int64) * 37) % cfg.T).astype(np.int32)
    want = np.zeros((rows, cfg.d))
    for g in range(G):
        sl = slice(int(offsets[g]), int(offsets[g + 1]))
        want[sl] = O.expert_ffn(inp.x[row_token[sl]], inp.w1[g], inp.w2[g], act,
                                w3=None if inp.w3 is None else inp.w3[g])
    return cfg, inp, offsets, row_token, want


def _call(cfg, inp, offsets, row_token, group_bound):
    dev = {k: to_torch(v, "cuda") for k, v in inp.tensors().items()}
    c = config_of(cfg)
    ws = torch.empty(M.moe_workspace_bytes(c), dtype=torch.uint8, device="cuda")
    rows = int(offsets[-1])
    y = torch.full((rows, cfg.d), 5.0, dtype=torch.float32, device="cuda")
    L.moe_expert_ffn(c, len(offsets) - 1, dev["x"], torch.from_numpy(row_token).cuda(),
                     torch.from_numpy(offsets).cuda(), rows, group_bound, dev["w1"],
                     dev.get("w3"), dev["w2"], None, None, y, 0, ws)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("act", ["swiglu", "relu"])
def test_group_above_32_rows_with_true_bound(act):
    require_gpu()
    sizes = (5, 40, 0, 17)
    banner(f"group_bound true: sizes={sizes} act={act}")
    cfg, inp, offsets, row_token, want = _setup(sizes, act)
    y = _call(cfg, inp, offsets, row_token, max(sizes))
    assert rel_l2(y, want) <= 2e-2
    assert worst_row_error(y, want) <= 5e-2


@pytest.mark.parametrize("act", ["swiglu", "relu"])
def test_understated_group_bound_poisons_that_group(act):
    require_gpu()
    sizes = (5, 40, 0, 17)
    banner(f"group_bound understated: sizes={sizes} act={act}")
    cfg, inp, offsets, row_token, want = _setup(sizes, act)
    y = _call(cfg, inp, offsets, row_token, 32)
    big = slice(int(offsets[1]), int(offsets[2]))
    assert np.all(np.isnan(y[big]))
    ok = np.ones(y.shape[0], bool)
    ok[big] = False
    assert np.all(np.isfinite(y[ok]))
    assert rel_l2(y[ok], want[ok]) <= 2e-2
    assert worst_row_error(y[ok], want[ok]) <= 5e-2
