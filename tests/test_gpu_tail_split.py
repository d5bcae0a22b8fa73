"""Tail split of the tiled expert GEMM (float32 down projection and gated up
projection).

When the last round of 256 x 256 output tiles would leave at least half the
persistent blocks idle, those tiles are cut into parts of their reduction and
finished afterwards: the down projection's later parts' partials (two or
three parts) are added to the output; the gated up projection's two halves
both write partials and a fixup applies silu(gate) * up.  These cases pick group sizes and row
bounds that make the split happen, both after whole rounds of tiles (w >= 1)
and with fewer tiles than half the launch (w = 0), and compare the staged
expert FFN (and the up projection's hidden rows) with the oracle's per group,
with biases and with accumulation into the output.
"""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_26_amd as M
from sparse_mixture_experts_26_amd import _lib as L
from sparse_mixture_experts_26_amd.layer import config_of
from tests.gpu_util import banner, host, rel_l2, require_gpu
from workloads import LayerConfig, make_inputs, to_torch

pytestmark = pytest.mark.gpu

BM = BR = 256  # output tile of the tiled kernel


def _split_expected(offsets, rows_bound, n_groups, N, K, cus, d=None, gated=False):
    """Whether the launch splits, from the documented plan (host-side mirror).
    A gated launch covers 128 output columns per tile; the split scratch is
    sized by the model width d (its tile count with 256-column tiles)."""
    sizes = np.diff(offsets)
    entries = int(sum((s + BM - 1) // BM for s in sizes))
    cols = BR // 2 if gated else BR
    n_tiles_n = (N + cols - 1) // cols
    max_entries = (rows_bound + BM - 1) // BM + n_groups
    P = min(cus, max_entries * n_tiles_n)
    tiles = entries * n_tiles_n
    w, r = divmod(tiles, P)
    width = N if d is None else d
    cap = min(128, max_entries * ((width + BR - 1) // BR))
    nk = (K + 63) // 64
    min_nk = 48 if gated else 2  # the gated form splits only deep reductions
    split = r > 0 and 2 * r <= P and r <= cap and nk >= min_nk
    parts = (3 if (not gated and 3 * r <= P and nk >= 3) else 2) if split else 1
    return split, w, r, P, parts


@pytest.mark.parametrize("sizes,rows_bound,d,h", [
    ((4200, 300), 4500, 4096, 256),   # 19 x 16 tiles on 256 blocks: one whole round, 48 in 3 parts
    ((5000, 400), 5400, 4096, 256),   # 22 x 16 tiles: one whole round, 96 in 2 parts
    ((300, 200), 4096, 512, 192),     # 3 x 2 tiles on a 36-block launch: every tile in 3 parts
    # ragged everywhere: 640 columns (2.5 column tiles) and a reduction of 200
    # (the second half ends in a partial stage)
    ((700, 50, 333), 4096, 640, 200),
])
def test_tail_split_matches_oracle(sizes, rows_bound, d, h):
    require_gpu()
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offsets[-1])
    # T = rows_bound tokens, so that moe_workspace_bytes covers the row bound
    T = rows_bound
    cfg = LayerConfig(name="tail_split", cfg_id=71, T=T, d=d, E=G, k=1, h=h, act="swiglu",
                      capacity_factor=0.0, dtype="bf16", ffn_bias=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    split, w, r, P, parts = _split_expected(offsets, rows_bound, G, d, h, cus)
    banner(f"tail split sizes={sizes} rows_bound={rows_bound} d={d} h={h} w={w} r={r} P={P} "
           f"parts={parts}")
    assert split, "case no longer exercises the split"
    inp = make_inputs(cfg, seed=3)
    # rows gather tokens in a scrambled order
    row_token = ((np.arange(rows, dtype=np.int64) * 7919) % T).astype(np.int32)
    dev = {k: to_torch(v, "cuda") for k, v in inp.tensors().items()}
    c = config_of(cfg)
    ws = torch.empty(M.moe_workspace_bytes(c), dtype=torch.uint8, device="cuda")
    off_d = torch.from_numpy(offsets).cuda()
    rt_d = torch.from_numpy(row_token).cuda()
    y = torch.empty(rows_bound, d, dtype=torch.float32, device="cuda")
    args = (c, G, dev["x"], rt_d, off_d, rows_bound, rows_bound, dev["w1"], dev["w3"], dev["w2"],
            dev["b1"], dev["b2"], y)
    L.moe_expert_ffn(*args, 0, ws)
    torch.cuda.synchronize()
    y1 = host(y)[:rows].copy()
    L.moe_expert_ffn(*args, 1, ws)  # accumulate: twice the result
    torch.cuda.synchronize()
    y2 = host(y)[:rows]
    want = np.zeros((rows, d))
    for g in range(G):
        sl = slice(int(offsets[g]), int(offsets[g + 1]))
        want[sl] = O.expert_ffn(inp.x[row_token[sl]], inp.w1[g], inp.w2[g], cfg.act,
                                w3=inp.w3[g], b1=inp.b1[g], b2=inp.b2[g])
    assert rel_l2(y1, want) <= 2e-2
    # the second call adds the same terms onto the first result (in another
    # float32 order for split tiles)
    assert rel_l2(y2, 2 * y1) <= 1e-6


@pytest.mark.parametrize("sizes,rows_bound,d,h", [
    ((4200, 300), 4500, 3072, 2048),  # 19 x 16 tiles on 256 blocks: one whole round, 48 split
    ((300, 200), 4096, 3072, 384),    # 3 x 3 tiles on a 54-block launch: every tile split
    # ragged: 200 hidden units (the second column tile is partial) and a
    # reduction of 3080 (the second half ends in a partial stage)
    ((700, 50, 333), 4096, 3080, 200),
])
def test_gated_up_tail_split_matches_oracle(sizes, rows_bound, d, h):
    """moe_expert_up (SwiGLU, with b1) at sizes whose launch splits its tail
    tiles: every hidden row against the oracle's silu(x W1^T + b1) * (x W3^T)."""
    require_gpu()
    from tests.gpu_util import worst_row_error
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offsets[-1])
    T = rows_bound
    cfg = LayerConfig(name="tail_split_up", cfg_id=72, T=T, d=d, E=G, k=1, h=h, act="swiglu",
                      capacity_factor=0.0, dtype="bf16", ffn_bias=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    split, w, r, P, _ = _split_expected(offsets, rows_bound, G, h, d, cus, d=d, gated=True)
    banner(f"gated up tail split sizes={sizes} rows_bound={rows_bound} d={d} h={h} w={w} r={r} "
           f"P={P}")
    assert split, "case no longer exercises the split"
    inp = make_inputs(cfg, seed=4)
    row_token = ((np.arange(rows, dtype=np.int64) * 7919) % T).astype(np.int32)
    dev = {k: to_torch(v, "cuda") for k, v in inp.tensors().items()}
    c = config_of(cfg)
    ws = torch.empty(M.moe_workspace_bytes(c), dtype=torch.uint8, device="cuda")
    off_d = torch.from_numpy(offsets).cuda()
    rt_d = torch.from_numpy(row_token).cuda()
    hidden = torch.full((rows_bound, h), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.moe_expert_up(c, G, dev["x"], rt_d, off_d, rows_bound, rows_bound, dev["w1"], dev["w3"],
                    dev["b1"], hidden, ws)
    torch.cuda.synchronize()
    got = host(hidden)[:rows].astype(np.float64)
    want = np.zeros((rows, h))
    for g in range(G):
        sl = slice(int(offsets[g]), int(offsets[g + 1]))
        xr = O.to_f64(inp.x[row_token[sl]])
        a = xr @ O.to_f64(inp.w1[g]).T + O.to_f64(inp.b1[g])
        u = xr @ O.to_f64(inp.w3[g]).T
        want[sl] = O.activation("swiglu", a, u)
    assert np.all(np.isfinite(got))
    assert rel_l2(got, want) <= 2e-2
    assert worst_row_error(got, want) <= 5e-2


@pytest.mark.parametrize("E,k,T,d,h,act,bias,S", [
    (48, 1, 2000, 512, 256, "swiglu", False, 0),  # 9 x 2 tiles on a 112-block launch: 3 parts
    (32, 2, 3000, 640, 320, "gelu", True, 0),     # 26 x 3 tiles (2.5 column tiles) on 168: 2 parts
    # two shared experts run as one group of 2h-deep tiles (8 row tiles):
    # that launch cuts its XCD ranges by depth and does not split
    (48, 1, 2000, 512, 256, "swiglu", False, 2),
])
def test_layer_call_bf16_rows_split(E, k, T, d, h, act, bias, S):
    """The single layer call of a bf16 layer keeps its expert rows in bf16; a
    down projection whose tail tiles split then writes every part's float32
    sums, and a fixup adds them in part order with the bias and rounds once.
    A strongly biased router concentrates the rows in a few experts, so the
    launch has far fewer tiles than its row bound allows and splits; every
    token's output is checked against the oracle (routing replayed).  With two
    shared experts the call's down projection runs them as one group whose
    reduction covers both (one output row per token), on XCD ranges cut by
    depth and without a tail split."""
    from tests.gpu_util import oracle_forward, row_tol, upload, weights_of, worst_row_error, y_tol
    from sparse_mixture_experts_26_amd.layer import MoeLayer
    require_gpu()
    cfg = LayerConfig(name=f"layer_split_E{E}_k{k}_S{S}", cfg_id=77, T=T, d=d, E=E, k=k, h=h,
                      act=act, capacity_factor=0.0, dtype="bf16", ffn_bias=bias,
                      router_bias="normal", router_bias_std=3.0, n_shared=S)
    inp = make_inputs(cfg, seed=0)
    want = oracle_forward(inp)
    # the down launch's split plan (host-side mirror; the layer's workspace
    # caps the split tiles at half its row bound's tiles)
    offsets = want["offsets"]
    R = min(T * k, E * T)
    t_tiles = (T + BM - 1) // BM
    # the down launch holds the two shared experts as one group (S_down = 1);
    # the split scratch is carved for the layer's S
    S_down = 1 if S == 2 else S
    max_entries = (R + BM - 1) // BM + E + S_down * t_tiles
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    entries = int(sum((n + BM - 1) // BM for n in np.diff(offsets))) + S_down * t_tiles
    n_cols = (d + BR - 1) // BR
    P = min(cus, max_entries * n_cols)
    w, r = divmod(entries * n_cols, P)
    cap = min(128, (((R + BM - 1) // BM + E + S * t_tiles) * n_cols + 1) // 2)
    parts = 3 if 3 * r <= P else 2
    banner(f"layer split E={E} k={k} T={T} d={d} h={h}: {entries} x {n_cols} tiles on {P} "
           f"blocks, r={r}, cap={cap}, parts={parts}")
    if S != 2:
        assert r > 0 and 2 * r <= P and r <= cap, "case no longer exercises the split"
    dev = upload(inp)
    layer = MoeLayer(cfg, weights_of(dev))
    layer.out["y"].fill_(float("nan"))
    got = layer.forward(dev["x"], None, torch.from_numpy(want["logits"]).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(host(got["offsets"]), offsets)
    y = host(got["y"]).astype(np.float64)
    err, worst = rel_l2(y, want["y"]), worst_row_error(y, want["y"])
    banner(f"layer split: y rel-L2 {err:.3e}, worst token {worst:.3e}")
    assert err <= y_tol(cfg) and worst <= row_tol(cfg), (err, worst)
