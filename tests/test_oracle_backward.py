"""Pins of the backward oracle to facts outside itself (no GPU).

The pages print no backward, so the gradients are pinned by what mathematics
fixes: central finite differences of the forward oracle's objective (itself
pinned to the pages' worked examples), closed forms where the layer reduces to
a linear map or the logits are uniform, and invariants of softmax backwards.
Every planted mistake at the end must fail at least one of these pins.
"""
import math

import numpy as np
import pytest
from scipy.special import erf, expit

import oracle as O
import oracle.moe_oracle_backward as B

RNG = np.random.default_rng


def _layer(seed, *, T=10, d=6, E=4, k=2, h=5, act="gelu", cf=1.0, bias=True, noise=True,
           router_bias=True, shared=0, gated=None):
    r = RNG(seed)
    gated = act == "swiglu" if gated is None else gated
    p = {
        "x": r.normal(size=(T, d)),
        "w_g": r.normal(scale=0.6, size=(E, d)),
        "w1": r.normal(scale=0.5, size=(E, h, d)),
        "w2": r.normal(scale=0.5, size=(E, d, h)),
    }
    if gated:
        p["w3"] = r.normal(scale=0.5, size=(E, h, d))
    if bias:
        p["b1"] = r.normal(scale=0.3, size=(E, h))
        p["b2"] = r.normal(scale=0.3, size=(E, d))
    if router_bias:
        p["b_g"] = r.normal(scale=0.3, size=(E,))
    if noise:
        p["w_noise"] = r.normal(scale=0.4, size=(E, d))
        p["eps"] = r.normal(size=(T, E))
    if shared:
        p["ws1"] = r.normal(scale=0.5, size=(shared, h, d))
        p["ws2"] = r.normal(scale=0.5, size=(shared, d, h))
        if gated:
            p["ws3"] = r.normal(scale=0.5, size=(shared, h, d))
    dy = r.normal(size=(T, d))
    return p, dict(k=k, act=act, capacity_factor=cf), dy


CASES = {
    "gelu_drops_noise": dict(seed=1, act="gelu", cf=0.75),
    "swiglu_shared": dict(seed=2, act="swiglu", cf=1.25, bias=False, noise=False, shared=2),
    "relu_top1": dict(seed=3, act="relu", k=1, E=5, cf=1.0, router_bias=False),
    "swiglu_reroute": dict(seed=4, act="swiglu", E=6, cf=0.8, bias=False, shared=1),
}


def _directional_fd(p, kw, dy, name, direction, g_aux, g_z, overflow, h=1e-6):
    def L(delta):
        q = dict(p)
        q[name] = p[name] + delta * direction
        return B.layer_loss(q.pop("x"), q.pop("w_g"), q.pop("w1"), q.pop("w2"), dy=dy,
                            g_aux=g_aux, g_z=g_z, overflow=overflow, **kw, **q)
    return (L(h) - L(-h)) / (2 * h)


@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_matches_finite_differences(case):
    """Every gradient's inner product with a random direction equals the
    central difference of the forward oracle's objective (B1), with the
    logits left unrounded so the map is smooth away from routing changes."""
    spec = dict(CASES[case])
    overflow = "reroute" if "reroute" in case else "drop"
    p, kw, dy = _layer(**spec)
    g_aux, g_z = 0.7, 0.3
    args = {n: v for n, v in p.items() if n not in ("x", "w_g", "w1", "w2")}
    grads = O.moe_backward(p["x"], p["w_g"], p["w1"], p["w2"], dy=dy, g_aux=g_aux, g_z=g_z,
                           overflow=overflow, exact_logits=True, **kw, **args)
    fwd = grads["fwd"]
    # the case really exercises drops / re-routing where it says so
    if case in ("gelu_drops_noise", "swiglu_reroute"):
        assert (fwd["counts"] > fwd["kept"]).any()
    if overflow == "reroute":
        assert (fwd["final_expert"] != fwd["idx"]).any()
    names = {"x": "dx", "w_g": "dw_g", "w1": "dw1", "w2": "dw2", "w3": "dw3", "b1": "db1",
             "b2": "db2", "b_g": "db_g", "w_noise": "dw_noise", "ws1": "dws1", "ws2": "dws2",
             "ws3": "dws3"}
    r = RNG(100)
    checked = 0
    for pname, gname in names.items():
        if pname not in p:
            continue
        V = r.normal(size=p[pname].shape)
        fd = _directional_fd(p, kw, dy, pname, V, g_aux, g_z, overflow)
        an = float(np.sum(grads[gname] * V))
        assert an == pytest.approx(fd, rel=1e-6, abs=1e-7), (pname, an, fd)
        checked += 1
    assert checked >= 6


def test_dense_linear_closed_form():
    """E = 1, k = 1, dropless, ReLU with every pre-activation positive: the
    layer is the linear map y = (x W1^T + b1) W2^T + b2 with gate 1, whose
    gradients are the textbook ones; the router gets nothing (the gate of a
    single selected expert is the constant 1 and L_aux = 1 is constant)."""
    r = RNG(7)
    T, d, h = 9, 5, 7
    x = r.uniform(0.1, 1.0, size=(T, d))
    w1 = r.uniform(0.1, 1.0, size=(1, h, d))
    b1 = r.uniform(0.1, 1.0, size=(1, h))
    w2 = r.normal(size=(1, d, h))
    b2 = r.normal(size=(1, d))
    w_g = r.normal(size=(1, d))
    dy = r.normal(size=(T, d))
    g = O.moe_backward(x, w_g, w1, w2, k=1, act="relu", capacity_factor=0.0, dy=dy, b1=b1,
                       b2=b2, g_aux=0.5)
    U = x @ w1[0].T + b1[0]
    assert (U > 0).all()
    np.testing.assert_allclose(g["dx"], dy @ w2[0] @ w1[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dw2"][0], dy.T @ U, rtol=1e-12)
    np.testing.assert_allclose(g["dw1"][0], (dy @ w2[0]).T @ x, rtol=1e-12)
    np.testing.assert_allclose(g["db1"][0], (dy @ w2[0]).sum(0), rtol=1e-12)
    np.testing.assert_allclose(g["db2"][0], dy.sum(0), rtol=1e-12)
    assert np.abs(g["dw_g"]).max() < 1e-12


def test_aux_grad_at_uniform_logits():
    """Equal logits give p = 1/E, so dL_aux/dH[t,j] = (f_j - 1/E) / T."""
    T, E = 6, 5
    f = np.array([0.4, 0.3, 0.2, 0.1, 0.0])
    G = B.aux_loss_logit_grad(np.full((T, E), 0.37), f)
    np.testing.assert_allclose(G, np.tile((f - 1 / E) / T, (T, 1)), rtol=0, atol=1e-15)


def test_z_grad_at_zero_logits():
    """H = 0: log-partition log E and p = 1/E, so dL_z/dH = 2 log(E) / (E T)."""
    T, E = 4, 8
    G = B.z_loss_logit_grad(np.zeros((T, E)))
    np.testing.assert_allclose(G, 2 * math.log(E) / (E * T), rtol=1e-14)
    assert B.z_loss(np.zeros((T, E))) == pytest.approx(math.log(E) ** 2, rel=1e-14)


def test_activation_derivatives_against_closed_values():
    """GELU'(0) = 1/2, GELU'(u) -> 1 and 0 in the tails, ReLU' is a step,
    silu'(0) = 1/2 and d/dv silu(u) v = silu(u)."""
    u = np.array([0.0, 8.0, -8.0])
    du, _ = B.activation_backward("gelu", u, None, np.ones(3))
    np.testing.assert_allclose(du, [0.5, 1.0, 0.0], atol=1e-12)
    du, _ = B.activation_backward("relu", np.array([-1.0, 2.0]), None, np.array([3.0, 3.0]))
    assert du.tolist() == [0.0, 3.0]
    du, dv = B.activation_backward("swiglu", np.array([0.0, 1.5]), np.array([2.0, 1.0]),
                                   np.ones(2))
    assert du[0] == pytest.approx(0.5 * 2.0)
    assert dv[1] == pytest.approx(1.5 * expit(1.5))


def test_logit_gradient_rows_sum_to_zero_without_z_loss():
    """The gate softmax backward and the aux-loss backward are softmax
    backwards: without the z-loss every token's dH sums to 0, so db_g sums to
    0 as well."""
    p, kw, dy = _layer(11, act="gelu", cf=0.75, T=14)
    args = {n: v for n, v in p.items() if n not in ("x", "w_g", "w1", "w2")}
    g = O.moe_backward(p["x"], p["w_g"], p["w1"], p["w2"], dy=dy, g_aux=1.3, **kw, **args)
    np.testing.assert_allclose(g["dH"].sum(axis=1), 0.0, atol=1e-12)
    assert abs(g["db_g"].sum()) < 1e-11


def test_fully_dropped_token_gets_router_gradient_only():
    """A token whose every assignment was dropped has zero gate gradients, and
    its dx is the router's share dH W_g (+ the noise path) alone (B4)."""
    p, kw, dy = _layer(12, act="gelu", cf=0.3, T=16, noise=False)
    args = {n: v for n, v in p.items() if n not in ("x", "w_g", "w1", "w2")}
    g = O.moe_backward(p["x"], p["w_g"], p["w1"], p["w2"], dy=dy, **kw, **args)
    lost = (g["fwd"]["dest"] < 0).all(axis=1)
    assert lost.any()
    assert np.all(g["dg"][lost] == 0.0)
    np.testing.assert_allclose(g["dx"][lost], g["dH"][lost] @ p["w_g"], rtol=1e-12, atol=1e-14)
    # its selected logits still receive gradient when some other slot of the
    # token survives; with every slot lost the gate path gives exactly zero
    np.testing.assert_allclose(g["dH"][lost], 0.0, atol=0)


# --- expert-choice routing ---------------------------------------------------------------

EC_CASES = {
    "ec_gelu_partial_noise": dict(seed=21, act="gelu", cf=0.5, E=4, k=2),
    "ec_swiglu_shared": dict(seed=22, act="swiglu", cf=1.0, E=5, k=2, bias=False, noise=False,
                             shared=1),
}


@pytest.mark.parametrize("case", sorted(EC_CASES))
def test_expert_choice_backward_matches_finite_differences(case):
    """Expert-choice gradients (EB1) against central differences of the
    expert-choice forward oracle's objective."""
    p, kw, dy = _layer(**EC_CASES[case])
    g_aux, g_z = 0.7, 0.3
    args = {n: v for n, v in p.items() if n not in ("x", "w_g", "w1", "w2")}
    grads = O.moe_backward_expert_choice(p["x"], p["w_g"], p["w1"], p["w2"], dy=dy, g_aux=g_aux,
                                         g_z=g_z, exact_logits=True, **kw, **args)
    covered = (grads["fwd"]["slot"] >= 0).sum(axis=1)
    assert (covered == 0).any() or (covered > 1).any()  # some token has 0 or several experts
    names = {"x": "dx", "w_g": "dw_g", "w1": "dw1", "w2": "dw2", "w3": "dw3", "b1": "db1",
             "b2": "db2", "b_g": "db_g", "w_noise": "dw_noise", "ws1": "dws1", "ws2": "dws2",
             "ws3": "dws3"}
    r = RNG(200)
    for pname, gname in names.items():
        if pname not in p:
            continue
        V = r.normal(size=p[pname].shape)

        def L(delta):
            q = dict(p)
            q[pname] = p[pname] + delta * V
            return B.layer_loss_expert_choice(q.pop("x"), q.pop("w_g"), q.pop("w1"), q.pop("w2"),
                                              dy=dy, g_aux=g_aux, g_z=g_z, **kw, **q)
        fd = (L(1e-6) - L(-1e-6)) / 2e-6
        an = float(np.sum(grads[gname] * V))
        assert an == pytest.approx(fd, rel=1e-6, abs=1e-7), (pname, an, fd)


def test_expert_choice_identical_experts_give_no_router_gradient():
    """C' = T and identical experts: y = (sum_e S[t,e]) FFN(x_t) = FFN(x_t)
    whatever the logits, so dS is the same for every expert, its softmax
    backward is 0, the load-balancing term vanishes (f = 1/E) and the router
    gets nothing; dx is the dense FFN's."""
    p, kw, dy = _layer(23, act="gelu", cf=2.0, E=3, k=2, noise=False, router_bias=False)
    p["w1"][:] = p["w1"][0]
    p["w2"][:] = p["w2"][0]
    p["b1"][:] = p["b1"][0]
    p["b2"][:] = p["b2"][0]
    args = {n: v for n, v in p.items() if n not in ("x", "w_g", "w1", "w2")}
    # unrounded scores, so that they sum to 1 exactly
    g = O.moe_backward_expert_choice(p["x"], p["w_g"], p["w1"], p["w2"], dy=dy, g_aux=0.9,
                                     exact_logits=True, **kw, **args)
    assert (g["fwd"]["slot"] >= 0).all()
    assert np.abs(g["dw_g"]).max() < 1e-12
    dense = O.expert_ffn_backward(p["x"], p["w1"][0], p["w2"][0], "gelu", dy, None, p["b1"][0],
                                  p["b2"][0])
    np.testing.assert_allclose(g["dx"], dense["dx"], rtol=1e-10, atol=1e-12)


def test_expert_choice_aux_gradient_vanishes():
    """Every expert holds C' rows, so f = 1/E and g_aux changes nothing."""
    p, kw, dy = _layer(24, act="relu", cf=0.75, E=4, k=2)
    args = {n: v for n, v in p.items() if n not in ("x", "w_g", "w1", "w2")}
    a = O.moe_backward_expert_choice(p["x"], p["w_g"], p["w1"], p["w2"], dy=dy, g_aux=0.0, **kw,
                                     **args)
    b = O.moe_backward_expert_choice(p["x"], p["w_g"], p["w1"], p["w2"], dy=dy, g_aux=5.0, **kw,
                                     **args)
    np.testing.assert_allclose(a["dw_g"], b["dw_g"], rtol=0, atol=1e-12)


# --- planted mistakes ------------------------------------------------------------------

def _gelu_no_density(act, u, v, dhid):
    if act == "gelu":
        return dhid * 0.5 * (1.0 + erf(u / math.sqrt(2.0))), None
    return ORIG_ACT(act, u, v, dhid)


def _swiglu_dv_wrong(act, u, v, dhid):
    if act == "swiglu":
        s = expit(u)
        return dhid * v * s * (1.0 + u * (1.0 - s)), dhid * v * s
    return ORIG_ACT(act, u, v, dhid)


def _gate_bwd_sign(g, dg):
    return g * (dg + (g * dg).sum(axis=1, keepdims=True))


def _gate_bwd_identity(g, dg):
    return np.asarray(dg, np.float64)


def _aux_grad_no_E(H, f):
    return ORIG_AUX(H, f) / np.asarray(H).shape[1]


def _z_grad_no_lse(H):
    return (2.0 / np.asarray(H).shape[0]) * O.full_softmax(H)


def _router_noise_no_sigmoid(x, w_g, dH, w_noise=None, eps=None):
    out = ORIG_ROUTER(x, w_g, dH, None, None)
    if w_noise is not None:
        dn = np.asarray(dH) * O.to_f64(eps)
        out["dw_noise"] = dn.T @ O.to_f64(x)
        out["dx"] = out["dx"] + dn @ O.to_f64(w_noise)
    return out


def _expert_bwd_transposed_dw2(*a, **kw):
    res = ORIG_EXPERT(*a, **kw)
    d, h = res["dw2"].shape
    if d == h:
        res["dw2"] = res["dw2"].T
    else:
        res["dw2"] = res["dw2"].T.reshape(d, h)
    return res


def _softmax_bwd_no_sum(p, dS):
    return np.asarray(p) * np.asarray(dS)


def _softmax_bwd_sign(p, dS):
    p = np.asarray(p)
    dS = np.asarray(dS)
    return p * (dS + (p * dS).sum(axis=1, keepdims=True))


ORIG_ACT = B.activation_backward
ORIG_AUX = B.aux_loss_logit_grad
ORIG_ROUTER = B.router_backward
ORIG_EXPERT = B.expert_ffn_backward

MUTATIONS = {
    "gelu_no_density": ("activation_backward", _gelu_no_density),
    "swiglu_dv_wrong": ("activation_backward", _swiglu_dv_wrong),
    "gate_bwd_sign": ("gate_softmax_backward", _gate_bwd_sign),
    "gate_bwd_identity": ("gate_softmax_backward", _gate_bwd_identity),
    "aux_grad_no_E": ("aux_loss_logit_grad", _aux_grad_no_E),
    "z_grad_no_lse": ("z_loss_logit_grad", _z_grad_no_lse),
    "router_noise_no_sigmoid": ("router_backward", _router_noise_no_sigmoid),
    "expert_dw2_transposed": ("expert_ffn_backward", _expert_bwd_transposed_dw2),
    "ec_softmax_bwd_no_sum": ("softmax_backward", _softmax_bwd_no_sum),
    "ec_softmax_bwd_sign": ("softmax_backward", _softmax_bwd_sign),
}

PINS = [
    lambda: [test_backward_matches_finite_differences(c) for c in sorted(CASES)],
    test_dense_linear_closed_form,
    test_aux_grad_at_uniform_logits,
    test_z_grad_at_zero_logits,
    test_activation_derivatives_against_closed_values,
    test_logit_gradient_rows_sum_to_zero_without_z_loss,
    test_fully_dropped_token_gets_router_gradient_only,
    lambda: [test_expert_choice_backward_matches_finite_differences(c) for c in sorted(EC_CASES)],
    test_expert_choice_identical_experts_give_no_router_gradient,
    test_expert_choice_aux_gradient_vanishes,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_backward_mistake(name, monkeypatch):
    fn_name, bad = MUTATIONS[name]
    monkeypatch.setattr(B, fn_name, bad)
    caught = False
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught = True
            break
    assert caught, f"no pin caught the mutation {name}"
