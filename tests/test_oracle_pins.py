"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test checks the oracle against something the pages print, a closed form,
an invariant, a library routine it must reduce to, or brute force on tiny
inputs.  Sources are cited by page title and section; the printed values live
in tests/golden/ with their citations.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from workloads import FULL, SMALL, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --- worked examples printed on the pages -------------------------------------------

def test_top2_worked_example():
    """'Mixture-of-experts Models', Level 2: scores [1.8, .4, 1.2, -.3], top-2."""
    g = golden("top2_worked_example.json")
    H = np.array([g["scores"]], np.float32)
    dec = g["print_decimals"]
    p = O.full_softmax(H)[0]
    assert np.array_equal(np.round(p, dec), np.array(g["printed_weights"]))
    idx = O.select_top_k(H, g["k"])[0]
    gates = O.selected_gates(H, idx[None, :])[0]
    # the page prints experts in ascending-weight order; compare as expert -> gate
    printed = dict(zip(g["printed_experts"], g["printed_renormalised"]))
    assert set(idx.tolist()) == set(printed)
    assert idx[0] == 0  # slot 0 holds the best expert
    for e, w in zip(idx, gates):
        assert round(float(w), dec) == printed[int(e)]
    # the moe_forward path reproduces the same numbers, and P of one token is p
    d = 4
    out = O.moe_forward(np.eye(1, d, dtype=np.float32), np.zeros((4, d), np.float32),
                        np.zeros((4, 8, d), np.float32), np.zeros((4, d, 8), np.float32),
                        k=2, act="relu", capacity_factor=0, logits=H)
    assert np.allclose(out["gates"][0], gates, rtol=0, atol=0)
    assert np.array_equal(np.round(out["prob_mean"], dec), np.array(g["printed_weights"]))


def test_capacity_worked_example():
    """'Mixture-of-experts Models', Level 2 capacity example: loads [3 2 1 2],
    overflow [1 0 0 0] at capacity 2; with T=8, k=1, E=4 the formula of the
    routing lab's Capacity panel gives C = floor(1.0 * 8 * 1 / 4) = 2."""
    g = golden("capacity_worked_example.json")
    a = np.array(g["assignments"], np.int32)[:, None]
    E = g["n_experts"]
    C = O.capacity(1.0, a.shape[0], 1, E)
    assert C == g["capacity"]
    disp = O.dispatch(a, E, C)
    assert disp["counts"].tolist() == g["printed_loads"]
    st = O.balance_stats(disp["counts"], disp["kept"], np.full(E, 1 / E), a.shape[0], 1, E)
    assert st["overflow"].tolist() == g["printed_overflow"]
    # arrival order: the third request for expert 0 (token 2) is the one dropped
    assert disp["dest"][:, 0].tolist() == [0, 1, -1, 2, 3, 4, 5, 6]
    rec = O.overflow_record(a, disp["dest"])
    assert rec == [{"token": 2, "selected": [0], "processed": [], "fallback": "drop",
                    "dropped": [0]}]
    assert st["drop_rate"] == pytest.approx(1 / 8)


def test_load_deviation_example():
    """'Mixture-of-experts Models', Level 3: loads [47,26,17,10] deviate by 46."""
    g = golden("load_deviation_example.json")
    loads = np.array(g["loads"])
    st = O.balance_stats(loads, loads, np.full(4, 0.25), T=100, k=1, E=4)
    assert st["deviation"] == g["printed_deviation"]


def test_load_cv_hand_worked_values():
    """The load coefficient of variation ('Mixture-of-experts Models', Level 3,
    asks for it or another stated imbalance measure; read as the population
    standard deviation of the per-expert counts over their mean), worked by
    hand on the loads the pages print:
      [47,26,17,10] (Level 3): mean 25, squared deviations 484+1+64+225 = 774,
        sqrt(774/4)/25 = 0.5564171...
      [3,2,1,2] (Level 2 capacity example): mean 2, squared deviations 2,
        sqrt(2/4)/2 = 0.3535533...
    A sample standard deviation would give 0.6425 and 0.4082; equal loads
    give 0."""
    cases = (([47, 26, 17, 10], math.sqrt(774 / 4) / 25, 0.5564171),
             ([3, 2, 1, 2], math.sqrt(0.5) / 2, 0.3535534),
             ([5, 5, 5, 5], 0.0, 0.0))
    for loads, exact, printed7 in cases:
        loads = np.array(loads)
        E = loads.size
        T = int(loads.sum())
        st = O.balance_stats(loads, loads, np.full(E, 1.0 / E), T=T, k=1, E=E)
        H = np.zeros((T, E), np.float32)
        dest = np.zeros((T, 1), np.int32)
        d = O.routing_diagnostics(H, loads, loads, dest, C=T, T=T, k=1, E=E)
        for v in (st["load_cv"], d["load_cv"]):
            assert v == pytest.approx(exact, rel=1e-12, abs=1e-15)
            assert round(v, 7) == pytest.approx(printed7, abs=1e-7)


# --- top-k and gates -------------------------------------------------------------

def _beats(H, a, b):
    return H[a] > H[b] or (H[a] == H[b] and a < b)


def test_topk_brute_force_with_ties_and_signed_zero():
    """Every row of {-1, -0.0, +0.0, 1}^4 and every k: the oracle's choice is the
    unique ordered k-tuple in which each slot beats the later slots and every
    unselected expert (value first, then lower index)."""
    vals = [-1.0, -0.0, 0.0, 1.0]
    rows = np.array(list(itertools.product(vals, repeat=4)), np.float32)
    for k in range(1, 5):
        idx = O.select_top_k(rows, k)
        for r, H in enumerate(rows):
            found = []
            for perm in itertools.permutations(range(4), k):
                rest = [e for e in range(4) if e not in perm]
                ok = all(_beats(H, perm[i], perm[j]) for i in range(k) for j in range(i + 1, k))
                ok = ok and all(_beats(H, p, q) for p in perm for q in rest)
                if ok:
                    found.append(perm)
            assert len(found) == 1
            assert tuple(idx[r]) == found[0], (H, k)


def test_gate_closed_forms():
    rng = np.random.default_rng(7)
    H = rng.standard_normal((50, 6)).astype(np.float32)
    # k = 1: gate exactly 1
    g1 = O.selected_gates(H, O.select_top_k(H, 1))
    assert np.all(g1 == 1.0)
    # k = E: gates are the full softmax in slot order
    idx = O.select_top_k(H, 6)
    gE = O.selected_gates(H, idx)
    assert np.allclose(gE, np.take_along_axis(O.full_softmax(H), idx.astype(np.int64), 1),
                       rtol=0, atol=1e-15)
    # any k: gates sum to 1, decrease along slots, and equal the renormalised
    # full-softmax probabilities ('Mixture-of-Experts & Sparse Model Scaling' lab 1)
    for k in (2, 3, 4):
        idx = O.select_top_k(H, k)
        g = O.selected_gates(H, idx)
        assert np.allclose(g.sum(1), 1.0, rtol=0, atol=1e-15)
        assert np.all(np.diff(g, axis=1) <= 0)
        p = np.take_along_axis(O.full_softmax(H), idx.astype(np.int64), 1)
        assert np.allclose(g, p / p.sum(1, keepdims=True), rtol=1e-14, atol=0)
    # softmax matches torch's on the same logits
    assert np.allclose(O.full_softmax(H), torch.softmax(torch.from_numpy(H).double(), 1).numpy(),
                       rtol=1e-14, atol=0)


# --- router ----------------------------------------------------------------------

def test_router_identity_rows_give_weight_columns():
    """With x = basis vectors, H[j, e] = W_g[e, j] (+ b_g[e]): pins the operand
    orientation x W_g^T of the router, including a non-square case."""
    rng = np.random.default_rng(3)
    E, d = 5, 7
    W = rng.standard_normal((E, d)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    H = O.router_logits(np.eye(d, dtype=np.float32), W, b_g=b)
    assert np.array_equal(H, (W.T.astype(np.float64) + b).astype(np.float32))


def test_router_noise_reduces_and_matches_softplus():
    """'LLM part 09' s.2: H = x W_g + eps * softplus(x W_noise).  eps = 0 gives
    the plain router; with basis-vector inputs the noise term is
    eps * log(1 + exp(W_noise^T)), checked against numpy's logaddexp."""
    rng = np.random.default_rng(4)
    E, d = 4, 6
    W = rng.standard_normal((E, d)).astype(np.float32)
    Wn = (3 * rng.standard_normal((E, d))).astype(np.float32)
    x = np.eye(d, dtype=np.float32)
    H0 = O.router_logits(x, W, w_noise=Wn, eps=np.zeros((d, E), np.float32))
    assert np.array_equal(H0, O.router_logits(x, W))
    eps = rng.standard_normal((d, E)).astype(np.float32)
    H = O.router_logits(x, W, w_noise=Wn, eps=eps)
    ref = W.T.astype(np.float64) + eps * np.logaddexp(0.0, Wn.T.astype(np.float64))
    assert np.allclose(H, ref.astype(np.float32), rtol=1e-6, atol=0)
    # softplus itself, including large |z|
    z = np.array([-800.0, -30.0, -1.0, 0.0, 1.0, 30.0, 800.0])
    assert np.allclose(O.softplus(z), np.logaddexp(0.0, z), rtol=1e-15, atol=0)
    tz = torch.nn.functional.softplus(torch.from_numpy(z[1:-1]), threshold=1e9).numpy()
    assert np.allclose(O.softplus(z[1:-1]), tz, rtol=1e-14, atol=0)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x0001, 0x7F7F], np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(O.to_f64(bits), want)


# --- capacity and dispatch -------------------------------------------------------

def test_capacity_formula_values():
    """'3D mixture-of-experts routing lab', Capacity: C = factor*tokens*k/experts,
    floored; at k = 1 it is 'LLM part 09' s.3's factor * T / E."""
    expect = {"toy_fp32": 40, "switch_top1": 32, "mixtral_decode": 32,
              "mixtral_prefill": 8192, "finegrained_shared": 1920, "mixtral_prefill_ec": 2048,
              "finegrained_reroute": 1920}
    for name, c in FULL.items():
        assert O.capacity(c.capacity_factor, c.T, c.k, c.E) == expect[name]
    assert O.capacity(1.25, 100, 1, 4) == 31       # floor, not round
    assert O.capacity(0.01, 10, 1, 4) == 0         # no clamp: everything drops
    # lab 3 of 'Mixture-of-Experts & Sparse Model Scaling' uses int(avg * factor)
    assert O.capacity(1.5, 100, 1, 4) == int(100 / 4 * 1.5)


def test_toy_layer_at_binding_capacities():
    """The toy layer again at capacity factors 1.0 and 0.5: C = 32 and 16 by
    the capacity formula, so with 128 assignments over 4 experts some must
    drop; the definitional arrival-order walk and the vectorised dispatch
    agree on which, every kept load is at most C, and a factor-0.5 layer
    keeps exactly 4 C rows (every expert is over-subscribed)."""
    for cf, C in ((1.0, 32), (0.5, 16)):
        cfg = FULL["toy_fp32"].with_(name=f"toy_cf{cf}", capacity_factor=cf)
        assert O.capacity(cf, cfg.T, cfg.k, cfg.E) == C
        inp = make_inputs(cfg, 0)
        H = O.router_logits(inp.x, inp.w_g, inp.b_g)
        idx = O.select_top_k(H, cfg.k)
        walk = O.dispatch_in_arrival_order(idx, cfg.E, C)
        vec = O.dispatch(idx, cfg.E, C)
        kept = np.diff(vec["offsets"])
        assert np.all(kept <= C)
        assert int(kept.sum()) < cfg.T * cfg.k
        assert np.array_equal(walk["slot_rank"] >= 0, vec["dest"] >= 0)
        assert np.array_equal(walk["kept"], kept)
        if cf == 0.5:
            assert int(kept.sum()) == 4 * C


def _all_idx_patterns(T, E, k):
    choices = list(itertools.permutations(range(E), k))
    for combo in itertools.product(choices, repeat=T):
        yield np.array(combo, np.int32).reshape(T, k)


@pytest.mark.parametrize("T,E,k", [(3, 3, 1), (3, 3, 2), (4, 3, 2), (2, 4, 3)])
def test_dispatch_brute_force(T, E, k):
    """Every routing pattern of tiny batches x three capacity factors: the
    vectorised dispatch equals the sequential arrival-order walk of lab 3."""
    for idx in _all_idx_patterns(T, E, k):
        for cf in (0.5, 1.0, 1.5):
            C = O.capacity(cf, T, k, E)
            seq = O.dispatch_in_arrival_order(idx, E, C)
            vec = O.dispatch(idx, E, C)
            assert np.array_equal(seq["counts"], vec["counts"])
            assert np.array_equal(seq["kept"], vec["kept"])
            assert np.array_equal(seq["slot_rank"], np.where(vec["dest"] >= 0, vec["rank"], -1))
            flat = idx.reshape(-1)
            want_dest = np.where(seq["slot_rank"].reshape(-1) >= 0,
                                 vec["offsets"][flat] + seq["slot_rank"].reshape(-1), -1)
            assert np.array_equal(vec["dest"].reshape(-1), want_dest)


def test_dispatch_invariants_random():
    """Lab 3 invariants (load never exceeds C; every assignment counted once)
    and the layout contract on a larger random case with heavy skew."""
    rng = np.random.default_rng(11)
    T, E, k = 500, 8, 3
    H = (rng.standard_normal((T, E)) + np.linspace(3, 0, E)).astype(np.float32)
    idx = O.select_top_k(H, k)
    for cf in (0.25, 1.0, 1.25, 0):
        C = O.capacity(cf, T, k, E)
        d = O.dispatch(idx, E, C)
        assert d["counts"].sum() == T * k
        assert np.all(d["kept"] <= C) and np.all(d["kept"] == np.minimum(d["counts"], C))
        assert d["offsets"][-1] == d["kept"].sum() == len(d["row_token"])
        kept_mask = d["dest"] >= 0
        assert kept_mask.sum() == d["kept"].sum()
        for t, s in zip(*np.nonzero(kept_mask)):
            r = d["dest"][t, s]
            e = idx[t, s]
            assert d["offsets"][e] <= r < d["offsets"][e + 1]
            assert d["row_token"][r] == t
        for e in range(E):  # rows of one expert are in arrival (token) order
            rt = d["row_token"][d["offsets"][e]:d["offsets"][e + 1]]
            assert np.all(np.diff(rt) > 0)
        if cf == 0:
            assert np.all(kept_mask)


def test_lab3_capacity_scenarios():
    """'Mixture-of-Experts & Sparse Model Scaling' lab 3: balanced routing with a
    generous factor drops under 5%; skewed routing with a tight factor drops
    more; no expert exceeds its capacity.  Own seeded draws, same scenario."""
    rng = np.random.default_rng(2)
    n, E = 100, 4
    bal = rng.integers(0, E, n).astype(np.int32)[:, None]
    skew = np.concatenate([np.zeros(60, np.int32), rng.integers(1, E, 40).astype(np.int32)])
    rng.shuffle(skew)
    skew = skew[:, None]
    Ca, Cb = O.capacity(1.5, n, 1, E), O.capacity(1.0, n, 1, E)
    a, b = O.dispatch(bal, E, Ca), O.dispatch(skew, E, Cb)
    rate = lambda d: 1 - d["kept"].sum() / n
    assert rate(a) < 0.05
    assert rate(b) > rate(a)
    assert a["kept"].max() <= Ca and b["kept"].max() <= Cb


# --- load-balance statistics -----------------------------------------------------

def test_laux_closed_forms():
    """'Mixture-of-Experts & Sparse Model Scaling', Mathematical Formulation:
    L = N * sum f_i P_i equals 1 when f = P = 1/N; with f uniform it equals
    sum P_i = 1 for any P.  It can fall below 1 (f = (2/3, 1/3), P = (.34, .66)
    gives 2 * (2/3*.34 + 1/3*.66) = 0.89333...), so no lower bound is asserted."""
    E, T, k = 8, 64, 2
    H = np.zeros((T, E), np.float32)
    idx = np.stack([np.arange(T) % E, (np.arange(T) + 1) % E], 1).astype(np.int32)
    d = O.dispatch(idx, E, O.capacity(0, T, k, E))
    P = O.full_softmax(H).mean(0)
    st = O.balance_stats(d["counts"], d["kept"], P, T, k, E)
    assert np.allclose(st["f"], 1 / E) and np.allclose(P, 1 / E)
    assert st["l_aux"] == pytest.approx(1.0, abs=1e-15)
    rng = np.random.default_rng(5)
    P2 = O.full_softmax(rng.standard_normal((T, E)).astype(np.float32)).mean(0)
    assert O.balance_stats(d["counts"], d["kept"], P2, T, k, E)["l_aux"] == pytest.approx(1.0, abs=1e-14)
    # the counterexample: three top-1 tokens over two experts
    probs = np.array([[.51, .49], [.51, .49], [0.0, 1.0]])
    counts = np.array([2, 1])
    st = O.balance_stats(counts, counts, probs.mean(0), T=3, k=1, E=2)
    assert st["l_aux"] == pytest.approx(2 * (2 / 3 * 0.34 + 1 / 3 * 0.66), abs=1e-15)
    assert st["l_aux"] < 1
    assert np.allclose(st["f"], [2 / 3, 1 / 3])


def test_lab2_collapse_detection():
    """'Mixture-of-Experts & Sparse Model Scaling' lab 2: with top-1 routing,
    balanced logits give L_aux < 1.5 and a collapse toward expert 0 (logit
    +5) gives L_aux > 1.5.  Own seeded draws of the same scenario."""
    rng = np.random.default_rng(10)
    n, E = 200, 6
    base = (0.5 * rng.standard_normal((n, E))).astype(np.float32)
    col = base.copy()
    col[:, 0] += 5.0

    def loss(H):
        idx = O.select_top_k(H, 1)
        d = O.dispatch(idx, E, O.capacity(0, n, 1, E))
        return O.balance_stats(d["counts"], d["kept"], O.full_softmax(H).mean(0), n, 1, E)["l_aux"]
    lb, lc = loss(base), loss(col)
    assert lb < lc and lc > 1.5 and lb < 1.5


# --- experts and the whole layer -------------------------------------------------

def test_activations_match_library_forms():
    a = np.linspace(-6, 6, 241)
    b = np.cos(a)
    ta, tb = torch.from_numpy(a), torch.from_numpy(b)
    F = torch.nn.functional
    assert np.allclose(O.activation("gelu", a), F.gelu(ta, approximate="none").numpy(), rtol=1e-14, atol=1e-16)
    assert np.array_equal(O.activation("relu", a), F.relu(ta).numpy())
    assert np.allclose(O.activation("swiglu", a, b), (F.silu(ta) * tb).numpy(), rtol=1e-14, atol=1e-16)


def _torch_ffn(x, w1, w2, act, w3=None, b1=None, b2=None):
    """Dense FFN through torch.nn.functional in float64 (nn.Linear convention)."""
    F = torch.nn.functional
    t = lambda a: None if a is None else torch.from_numpy(O.to_f64(a))
    xx = t(x)
    a = F.linear(xx, t(w1), t(b1))
    if act == "gelu":
        hid = F.gelu(a, approximate="none")
    elif act == "relu":
        hid = F.relu(a)
    else:
        hid = F.silu(a) * F.linear(xx, t(w3))
    return F.linear(hid, t(w2), t(b2)).numpy()


@pytest.mark.parametrize("act", ["gelu", "relu", "swiglu"])
def test_dense_equivalence_E1_k1(act):
    """E = 1, k = 1: the gate is exactly 1 and C = floor(1.0*T) = T, so the
    layer is the dense FFN: bit-identical to the oracle's own expert applied to
    all rows, and equal to torch's dense FFN within float64 rounding."""
    rng = np.random.default_rng(1)
    T, d, h = 37, 12, 20
    x = rng.standard_normal((T, d)).astype(np.float32)
    w1 = (0.3 * rng.standard_normal((1, h, d))).astype(np.float32)
    w3 = (0.3 * rng.standard_normal((1, h, d))).astype(np.float32) if act == "swiglu" else None
    w2 = (0.3 * rng.standard_normal((1, d, h))).astype(np.float32)
    b1 = (0.1 * rng.standard_normal((1, h))).astype(np.float32)
    b2 = (0.1 * rng.standard_normal((1, d))).astype(np.float32)
    wg = rng.standard_normal((1, d)).astype(np.float32)
    out = O.moe_forward(x, wg, w1, w2, w3=w3, b1=b1, b2=b2, k=1, act=act, capacity_factor=1.0)
    assert out["capacity"] == T and np.all(out["dest"] >= 0)
    dense = O.expert_ffn(x, w1[0], w2[0], act, None if w3 is None else w3[0], b1[0], b2[0])
    assert np.array_equal(out["y"], dense)
    ref = _torch_ffn(x, w1[0], w2[0], act, None if w3 is None else w3[0], b1[0], b2[0])
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-13)


def test_identical_experts_and_drops():
    """Identical experts: with nothing dropped the gates sum to 1 so y = FFN(x);
    when one of a token's slots is dropped, y = (surviving gate) * FFN(x), the
    gates are not rescaled; at C = 0 every token outputs zero."""
    rng = np.random.default_rng(2)
    T, d, h, E, k = 40, 8, 16, 4, 2
    x = rng.standard_normal((T, d)).astype(np.float32)
    one1 = (0.3 * rng.standard_normal((h, d))).astype(np.float32)
    one2 = (0.3 * rng.standard_normal((d, h))).astype(np.float32)
    w1 = np.repeat(one1[None], E, 0)
    w2 = np.repeat(one2[None], E, 0)
    wg = rng.standard_normal((E, d)).astype(np.float32)
    ref = _torch_ffn(x, one1, one2, "gelu")
    full = O.moe_forward(x, wg, w1, w2, k=k, act="gelu", capacity_factor=0)
    assert np.allclose(full["y"], ref, rtol=1e-12, atol=1e-13)
    tight = O.moe_forward(x, wg, w1, w2, k=k, act="gelu", capacity_factor=0.5)
    assert tight["capacity"] == 10  # floor(0.5 * 40 * 2 / 4)
    g = tight["gates"]
    kept = tight["dest"] >= 0
    scale = (g * kept).sum(1)
    assert np.any((scale > 0) & (scale < 1 - 1e-9))
    assert np.allclose(tight["y"], scale[:, None] * ref, rtol=1e-12, atol=1e-13)
    zero = O.moe_forward(x, wg, w1, w2, k=k, act="gelu", capacity_factor=1e-6)
    assert zero["capacity"] == 0 and np.all(zero["y"] == 0)
    assert zero["drop_rate"] == 1.0


def test_shared_experts_add_with_weight_one():
    """Shared experts ('Mixture-of-Experts & Sparse Model Scaling', Advanced
    Theory): every token, weight 1, never dropped; with C = 0 the layer output
    is exactly the sum of the shared experts' dense FFNs."""
    rng = np.random.default_rng(8)
    T, d, h, E, S = 30, 8, 12, 4, 2
    x = rng.standard_normal((T, d)).astype(np.float32)
    mk = lambda *s: (0.3 * rng.standard_normal(s)).astype(np.float32)
    w1, w3, w2 = mk(E, h, d), mk(E, h, d), mk(E, d, h)
    ws1, ws3, ws2 = mk(S, h, d), mk(S, h, d), mk(S, d, h)
    wg = mk(E, d)
    out = O.moe_forward(x, wg, w1, w2, w3=w3, ws1=ws1, ws3=ws3, ws2=ws2, k=2,
                        act="swiglu", capacity_factor=1e-9)
    ref = sum(_torch_ffn(x, ws1[s], ws2[s], "swiglu", ws3[s]) for s in range(S))
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-13)


def test_token_sampling_matches_full_run():
    cfg = SMALL["finegrained_small"].with_(T=200)
    inp = make_inputs(cfg)
    kw = dict(k=cfg.k, act=cfg.act, capacity_factor=cfg.capacity_factor, w3=inp.w3,
              b_g=inp.b_g, ws1=inp.ws1, ws3=inp.ws3, ws2=inp.ws2)
    full = O.moe_forward(inp.x, inp.w_g, inp.w1, inp.w2, **kw)
    toks = np.array([0, 3, 77, 199])
    part = O.moe_forward(inp.x, inp.w_g, inp.w1, inp.w2, tokens=toks, **kw)
    # BLAS may block a smaller product differently: equal to float64 rounding
    assert np.allclose(part["y"], full["y"][toks], rtol=1e-12, atol=1e-14)
    assert np.array_equal(part["dest"], full["dest"])


def test_small_configs_route_as_designed():
    """The reduced workloads keep the regimes of the full ones: drops where a
    capacity factor is set, none where dropless, noise in the Switch layer."""
    for name, cfg in SMALL.items():
        inp = make_inputs(cfg, experts=False)
        H = O.router_logits(inp.x, inp.w_g, inp.b_g, inp.w_noise, inp.eps)
        idx = O.select_top_k(H, cfg.k)
        C = O.capacity(cfg.capacity_factor, cfg.T, cfg.k, cfg.E)
        d = O.dispatch(idx, cfg.E, C)
        drops = int((d["counts"] - d["kept"]).sum())
        if cfg.dropless:
            assert drops == 0, name
        elif name != "toy_fp32":
            assert drops > 0, name


# --- router z-loss and routing diagnostics --------------------------------------

def _diag(H, idx_or_assign, C, k):
    H = np.asarray(H, np.float32)
    T, E = H.shape
    idx = np.asarray(idx_or_assign, np.int32).reshape(T, k)
    disp = O.dispatch(idx, E, C)
    return O.routing_diagnostics(H, disp["counts"], disp["kept"], disp["dest"], C, T, k, E)


def test_zloss_and_entropy_closed_forms():
    """Z1 on logits whose log-partition and entropy are known in closed form."""
    T, E = 5, 8
    d = _diag(np.zeros((T, E)), np.zeros((T, 1)), T, 1)
    assert d["z_loss"] == pytest.approx(math.log(E) ** 2, rel=1e-12)
    assert d["entropy"] == pytest.approx(math.log(E), rel=1e-12)   # uniform router
    d = _diag(np.full((T, E), 3.0), np.zeros((T, 1)), T, 1)
    assert d["z_loss"] == pytest.approx((3.0 + math.log(E)) ** 2, rel=1e-12)
    # two experts: entropy of a Bernoulli(sigmoid(a - b)); log-partition log(e^a + e^b)
    a, b = 1.5, -0.5
    q = 1 / (1 + math.exp(-(a - b)))
    d = _diag([[a, b]], [[0]], 1, 1)
    assert d["entropy"] == pytest.approx(-(q * math.log(q) + (1 - q) * math.log(1 - q)), rel=1e-12)
    assert d["z_loss"] == pytest.approx(math.log(math.exp(a) + math.exp(b)) ** 2, rel=1e-12)
    # one expert: the log-partition is the logit itself
    h = np.array([[0.5], [-2.0], [4.0]])
    d = _diag(h, np.zeros((3, 1)), 3, 1)
    assert d["z_loss"] == pytest.approx(np.mean(h ** 2), rel=1e-12)
    assert d["entropy"] == 0.0
    # a nearly one-hot router has almost no entropy
    d = _diag([[40.0, 0.0, 0.0]], [[0]], 1, 1)
    assert d["entropy"] < 1e-15


def test_diagnostics_on_the_capacity_worked_example():
    """'Mixture-of-experts Models', Level 2: assignments [0,0,0,1,1,2,3,3] with
    capacity 2 overflow expert 0 by one (printed [1 0 0 0]); that token loses
    its only assignment."""
    g = golden("capacity_worked_example.json")
    a = np.array(g["assignments"])
    H = np.zeros((a.size, 4), np.float32)
    d = _diag(H, a[:, None], g["capacity"], 1)
    assert d["overflow"].tolist() == g["printed_overflow"]
    assert d["overflow_total"] == 1
    assert d["utilisation"].tolist() == [1.0, 1.0, 0.5, 1.0]
    assert d["tokens_fully_dropped"] == 1 / 8 and d["tokens_partly_dropped"] == 0.0
    assert d["peak_to_mean"] == 3 / 2
    assert d["deviation"] == 1 + 0 + 1 + 0        # |3-2| + |2-2| + |1-2| + |2-2|


def test_diagnostics_partial_drops_with_two_slots():
    # k = 2, E = 2, C = 1: token 0 keeps both slots, token 1 loses both
    H = np.array([[1.0, 0.0], [1.0, 0.0]], np.float32)
    d = _diag(H, [[0, 1], [0, 1]], 1, 2)
    assert d["tokens_fully_dropped"] == 0.5 and d["tokens_partly_dropped"] == 0.0
    # C = 1, E = 3, k = 2 in arrival order: token 0 keeps experts 0 and 1,
    # token 1 finds expert 1 full and keeps 2, token 2 finds 2 and 0 full
    H = np.zeros((3, 3), np.float32)
    d = _diag(H, [[0, 1], [1, 2], [2, 0]], 1, 2)
    assert d["tokens_partly_dropped"] == 1 / 3 and d["tokens_fully_dropped"] == 1 / 3
