"""Pins of the oracle's expert-choice routing (CPU only).

"Mixture-of-Experts & Sparse Model Scaling", Advanced Theory & Extensions:
each expert takes the tokens it scores highest, up to its capacity, so every
expert is full and a token may be taken by no expert or by several.  The page
prints no example, so the pins are a hand-worked case, closed forms and an
independent brute force (repeated argmax instead of a sort).
"""
import itertools

import numpy as np
import pytest

import oracle as O
from workloads import LayerConfig, make_inputs


def _hand_logits():
    # softmax rows: t0 (0.731, 0.269), t1 (0.269, 0.731), t2 (0.881, 0.119), t3 (0.5, 0.5)
    return np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 0.0], [0.5, 0.5]], np.float32)


def test_ec_hand_example():
    S = O.expert_choice_scores(_hand_logits())
    assert np.allclose(S[:, 0], [0.7310586, 0.26894143, 0.8807971, 0.5], atol=1e-7)
    assert np.allclose(S.sum(1), 1.0, atol=1e-7)
    two = O.expert_choice_select(S, 2)
    # expert 0: t2 (0.881), t0 (0.731); expert 1: t1 (0.731), t3 (0.5) -- rows in token order
    assert two["row_token"].tolist() == [0, 2, 1, 3]
    assert two["offsets"].tolist() == [0, 2, 4]
    assert two["slot"].tolist() == [[0, -1], [-1, 2], [1, -1], [-1, 3]]
    one = O.expert_choice_select(S, 1)
    assert one["row_token"].tolist() == [2, 1]
    assert (one["slot"] >= 0).any(1).tolist() == [False, True, True, False]


def test_ec_ranks_on_scores_not_logits():
    # expert 0's logit is higher for t0 (2 > 1), its score higher for t1
    H = np.array([[2.0, 2.0], [1.0, 0.0]], np.float32)
    sel = O.expert_choice_select(O.expert_choice_scores(H), 1)
    assert sel["row_token"].tolist() == [1, 0]


def test_ec_uniform_scores_take_lowest_indices():
    for T, E, C in [(7, 3, 4), (5, 5, 1), (6, 2, 6)]:
        sel = O.expert_choice_select(O.expert_choice_scores(np.zeros((T, E), np.float32)), C)
        assert sel["row_token"].tolist() == list(range(min(C, T))) * E


def _repeated_argmax(S, C):
    """Independent selection: C rounds of argmax over the untaken tokens
    (np.argmax returns the first maximum, i.e. the lowest index on ties)."""
    T, E = S.shape
    out = []
    for e in range(E):
        col = S[:, e].astype(np.float64).copy()
        picked = []
        for _ in range(min(C, T)):
            t = int(np.argmax(col))
            picked.append(t)
            col[t] = -np.inf
        out.append(sorted(picked))
    return out


@pytest.mark.parametrize("T,E", [(4, 2), (3, 3)])
def test_ec_brute_force_with_ties(T, E):
    for vals in itertools.product([-1.0, 0.0, 1.0], repeat=T * E):
        H = np.array(vals, np.float32).reshape(T, E)
        S = O.expert_choice_scores(H)
        for C in range(0, T + 2):
            sel = O.expert_choice_select(S, C)
            want = _repeated_argmax(S, C)
            Cp = min(C, T)
            for e in range(E):
                assert sel["row_token"][e * Cp:(e + 1) * Cp].tolist() == want[e]
            # slot is the inverse of row_token
            for r, t in enumerate(sel["row_token"]):
                assert sel["slot"][t, r // Cp] == r


def _cfg(**kw):
    base = dict(name="ec", cfg_id=950, T=40, d=24, E=4, k=2, h=32, act="swiglu",
                capacity_factor=1.0, dtype="f32")
    base.update(kw)
    return LayerConfig(**base)


def _ec(inp, cfg, **kw):
    return O.moe_forward_expert_choice(
        inp.x, inp.w_g, inp.w1, inp.w2, k=cfg.k, act=cfg.act, capacity_factor=cfg.capacity_factor,
        w3=inp.w3, b_g=inp.b_g, b1=inp.b1, b2=inp.b2, ws1=inp.ws1, ws3=inp.ws3, ws2=inp.ws2, **kw)


def _identical_experts(inp):
    for name in ("w1", "w3", "w2"):
        w = getattr(inp, name)
        if w is not None:
            w[:] = w[0]


def test_ec_every_expert_full_and_stats():
    cfg = _cfg()
    inp = make_inputs(cfg, 1)
    out = _ec(inp, cfg)
    C = O.capacity(cfg.capacity_factor, cfg.T, cfg.k, cfg.E)
    assert C == 20 and out["counts"].tolist() == [20] * 4
    assert np.allclose(out["f"], 0.25)
    assert abs(out["l_aux"] - 1.0) < 1e-12  # E * sum(f P) = sum(P) = 1
    covered = (out["slot"] >= 0).any(1)
    assert out["drop_rate"] == pytest.approx(1 - covered.mean())
    assert np.all(out["y"][~covered] == 0)


def test_ec_full_capacity_identical_experts_is_the_dense_ffn():
    # C >= T: every expert takes every token, the scores of a token sum to 1
    cfg = _cfg(capacity_factor=4.0, act="gelu")
    inp = make_inputs(cfg, 2)
    _identical_experts(inp)
    out = _ec(inp, cfg)
    assert out["capacity_used"] == cfg.T and out["drop_rate"] == 0.0
    dense = O.expert_ffn(inp.x, inp.w1[0], inp.w2[0], "gelu")
    assert np.abs(out["y"] - dense).max() <= 1e-6 * np.abs(dense).max()


def test_ec_single_expert_is_exactly_dense():
    cfg = _cfg(E=1, k=1, capacity_factor=1.0)
    inp = make_inputs(cfg, 3)
    out = _ec(inp, cfg)
    assert np.all(out["scores"] == 1.0)
    dense = O.expert_ffn(inp.x, inp.w1[0], inp.w2[0], "swiglu", inp.w3[0])
    assert np.array_equal(out["y"], dense)


def test_ec_partial_coverage_gates_are_raw_scores():
    # identical experts: y_t = (sum of t's scores over the experts that took t) * FFN(x_t)
    cfg = _cfg(capacity_factor=0.5)
    inp = make_inputs(cfg, 4)
    _identical_experts(inp)
    out = _ec(inp, cfg)
    dense = O.expert_ffn(inp.x, inp.w1[0], inp.w2[0], "swiglu", inp.w3[0])
    took = out["slot"] >= 0
    w = (out["scores"].astype(np.float64) * took).sum(1)
    assert took.any(1).sum() < cfg.T  # some tokens are taken by no expert
    assert np.allclose(out["y"], w[:, None] * dense, rtol=1e-12, atol=1e-15)


def test_ec_capacity_above_batch_and_zero():
    cfg = _cfg(capacity_factor=10.0)
    inp = make_inputs(cfg, 5)
    out = _ec(inp, cfg)
    assert out["capacity_used"] == cfg.T
    cfg0 = _cfg(capacity_factor=1e-6, n_shared=1)
    inp0 = make_inputs(cfg0, 5)
    out0 = _ec(inp0, cfg0)
    assert out0["capacity_used"] == 0 and out0["drop_rate"] == 1.0
    assert np.array_equal(out0["y"], out0["shared"])
