"""CPU oracle for the backward pass of one sparse Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or call this module; the HIP
library never does, and nothing here is a fallback for it.

Plain NumPy, float64, the chain rule written out step by step over the forward
of ``moe_oracle`` (whose page citations and readings R1-R8, RR1-RR4, Z1 hold
here too).  The pages train these layers but print no backward formulas
([MoE&SMS] "Mathematical Formulation": the router is learned through the
gate values, and the balancing loss is differentiable through P_i while f_i is
a hard count; [LLM-09] s.4 the same; [MoEM] Level 2: routing decisions are
discrete).  Readings:
  B1  The layer's training objective is L = <dy, y> + g_aux * L_aux + g_z * L_z:
      dy [T,d] is the upstream gradient of the output, g_aux and g_z the
      weights of the load-balancing loss (R5) and of the z-loss (Z1).
  B2  Routing decisions -- the top-k set, the capacity drops, re-routing --
      and the counts f_i are piecewise constant: no gradient flows through
      them.  Gradients flow through the gates (R1), through P_i (R5) and
      through the log-partition of the z-loss (Z1).
  B3  The float32 rounding of the logits is treated as the identity.
  B4  A dropped slot still takes part in the softmax over the selected logits
      (its gate is not renormalised away, R4), so its logit receives gradient
      through the other slots' gates; its own gate gradient is zero.  A
      re-routed slot's gate gradient is dy . (output of the expert that
      processed it) (RR3).
  B5  Shared experts see every token with weight 1 and no router (R7).
  B6  Noise (R6) is a supplied input: eps gets no gradient, W_noise gets the
      gradient through softplus, whose derivative is the logistic sigmoid.
  B7  Every gradient is returned in float64; the library returns float32.
Expert-choice routing (EC1-EC6) adds one reading:
  EB1 The scores are the full softmax of the logits (their float32 rounding
      taken as the identity, B3) and the experts' token choices carry no
      gradient (B2), so the logits receive the full-softmax backward of
      dS[t,e] = dy_t . FFN_e(x_t) over the pairs some expert took (0 for the
      rest).  With every expert holding C' rows, f_i = 1/E and the
      load-balancing term's logit gradient vanishes.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf, expit

from .moe_oracle import activation, full_softmax, moe_forward, moe_forward_expert_choice, to_f64

__all__ = [
    "activation_backward", "expert_ffn_backward", "gate_softmax_backward",
    "aux_loss_logit_grad", "z_loss", "z_loss_logit_grad", "router_backward",
    "layer_loss", "moe_backward", "softmax_backward", "layer_loss_expert_choice",
    "moe_backward_expert_choice",
]


def activation_backward(act: str, u: np.ndarray, v: np.ndarray | None, dhid: np.ndarray):
    """Gradient of the hidden layer hid = act(u[, v]) (R8) with respect to its
    inputs, given dhid = dL/dhid.  Returns (du, dv); dv is None unless SwiGLU.

      GELU   hid = u Phi(u):         du = dhid (Phi(u) + u phi(u))
      ReLU   hid = max(u, 0):        du = dhid [u > 0]
      SwiGLU hid = u sigma(u) v:     du = dhid v sigma(u) (1 + u (1 - sigma(u))),
                                     dv = dhid u sigma(u)
    with Phi, phi the standard normal CDF and density and sigma the logistic
    function.
    """
    if act == "gelu":
        cdf = 0.5 * (1.0 + erf(u / math.sqrt(2.0)))
        pdf = np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)
        return dhid * (cdf + u * pdf), None
    if act == "relu":
        return dhid * (u > 0.0), None
    if act == "swiglu":
        s = expit(u)
        return dhid * v * s * (1.0 + u * (1.0 - s)), dhid * u * s
    raise ValueError(act)


def expert_ffn_backward(x_rows, w1, w2, act, dy_rows, w3=None, b1=None, b2=None) -> dict:
    """One expert FFN y = act(x W1^T + b1 [, x W3^T]) W2^T + b2 over a set of
    rows, and the gradients of sum(dy_rows * y) with respect to its rows and
    its weights.  dy_rows already carries each row's gate (the combine
    multiplies the expert output by it)."""
    x = to_f64(x_rows)
    dyr = np.asarray(dy_rows, np.float64)
    W1, W2 = to_f64(w1), to_f64(w2)
    u = x @ W1.T
    if b1 is not None:
        u = u + to_f64(b1)[None, :]
    v = x @ to_f64(w3).T if w3 is not None else None
    hid = activation(act, u, v)
    y = hid @ W2.T
    if b2 is not None:
        y = y + to_f64(b2)[None, :]
    # y = hid W2^T + b2
    dw2 = dyr.T @ hid
    db2 = dyr.sum(axis=0)
    dhid = dyr @ W2
    du, dv = activation_backward(act, u, v, dhid)
    # u = x W1^T + b1, v = x W3^T
    dw1 = du.T @ x
    db1 = du.sum(axis=0)
    dx = du @ W1
    dw3 = None
    if dv is not None:
        dw3 = dv.T @ x
        dx = dx + dv @ to_f64(w3)
    return {"y": y, "dx": dx, "dw1": dw1, "dw3": dw3, "dw2": dw2, "db1": db1, "db2": db2,
            "u": u, "v": v, "hid": hid}


def gate_softmax_backward(g: np.ndarray, dg: np.ndarray) -> np.ndarray:
    """Gates are the softmax over the k selected logits (R1): the selected
    logit s receives g_s (dg_s - sum_m g_m dg_m)."""
    g = np.asarray(g, np.float64)
    dg = np.asarray(dg, np.float64)
    return g * (dg - (g * dg).sum(axis=1, keepdims=True))


def aux_loss_logit_grad(H, f) -> np.ndarray:
    """dL_aux/dH for L_aux = E sum_i f_i P_i, P_i = mean_t softmax(H_t)_i (R5)
    with f held constant (B2):
      dL_aux/dH[t,j] = (E/T) p_tj (f_j - sum_i f_i p_ti)."""
    p = full_softmax(H)
    T, E = p.shape
    f = np.asarray(f, np.float64)
    return (E / T) * p * (f[None, :] - (p * f[None, :]).sum(axis=1, keepdims=True))


def _log_partition(H) -> np.ndarray:
    H = np.asarray(H, np.float64)
    m = H.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(H - m).sum(axis=1, keepdims=True)))[:, 0]


def z_loss(H) -> float:
    """Z1: mean over tokens of the squared log-partition of the logits."""
    return float(np.mean(_log_partition(H) ** 2))


def z_loss_logit_grad(H) -> np.ndarray:
    """dL_z/dH[t,j] = (2/T) lse_t p_tj (the derivative of the log-partition is
    the softmax)."""
    lse = _log_partition(H)
    p = full_softmax(H)
    return (2.0 / p.shape[0]) * lse[:, None] * p


def router_backward(x, w_g, dH, w_noise=None, eps=None) -> dict:
    """Gradients through H = x W_g^T + b_g + eps * softplus(x W_noise^T) (R6,
    B3, B6) given dH = dL/dH [T,E]."""
    x64 = to_f64(x)
    dH = np.asarray(dH, np.float64)
    out = {"dx": dH @ to_f64(w_g), "dw_g": dH.T @ x64, "db_g": dH.sum(axis=0), "dw_noise": None}
    if w_noise is not None:
        n = x64 @ to_f64(w_noise).T
        dn = dH * to_f64(eps) * expit(n)   # d softplus(n)/dn = sigmoid(n)
        out["dw_noise"] = dn.T @ x64
        out["dx"] = out["dx"] + dn @ to_f64(w_noise)
    return out


def layer_loss(x, w_g, w1, w2, *, k: int, act: str, capacity_factor: float, dy,
               g_aux: float = 0.0, g_z: float = 0.0, exact_logits: bool = True,
               **kw) -> float:
    """The objective of B1 evaluated by the forward oracle (derivative checks)."""
    fwd = moe_forward(x, w_g, w1, w2, k=k, act=act, capacity_factor=capacity_factor,
                      exact_logits=exact_logits, **kw)
    L = float(np.sum(np.asarray(dy, np.float64) * fwd["y"]))
    L += g_aux * fwd["l_aux"]
    L += g_z * z_loss(fwd["logits"])
    return L


def moe_backward(x, w_g, w1, w2, *, k: int, act: str, capacity_factor: float, dy,
                 g_aux: float = 0.0, g_z: float = 0.0, w3=None, b_g=None, w_noise=None,
                 eps=None, b1=None, b2=None, ws1=None, ws3=None, ws2=None, logits=None,
                 overflow: str = "drop", exact_logits: bool = False) -> dict:
    """Gradients of L (B1) with respect to x and every parameter, in float64.

    1. the forward's routing (top-k, gates, dispatch: held fixed, B2);
    2. every expert on its rows with the gate-weighted upstream rows g * dy_t:
       its weight gradients, its input gradients summed back to the tokens,
       and its outputs;
    3. shared experts with weight 1 (B5);
    4. gate gradients dg[t,s] = dy_t . (expert output of slot s), 0 for a
       dropped slot (B4);
    5. logit gradients: the selected-softmax backward scattered to the chosen
       experts, plus g_aux dL_aux/dH and g_z dL_z/dH;
    6. the router's parameters and its share of dx (B6).
    """
    fwd = moe_forward(x, w_g, w1, w2, k=k, act=act, capacity_factor=capacity_factor, w3=w3,
                      b_g=b_g, w_noise=w_noise, eps=eps, b1=b1, b2=b2, logits=logits,
                      overflow=overflow, exact_logits=exact_logits)
    H = np.asarray(fwd["logits"], np.float64)
    idx = np.asarray(fwd["idx"], np.int64)
    g = np.asarray(fwd["gates"], np.float64)
    dest = np.asarray(fwd["dest"], np.int64)
    offsets = np.asarray(fwd["offsets"], np.int64)
    row_token = np.asarray(fwd["row_token"], np.int64)
    xs = np.asarray(x)
    T, d = xs.shape
    E = np.asarray(w_g).shape[0]
    dy = np.asarray(dy, np.float64)

    R = int(offsets[-1])
    row_gate = np.zeros(R)
    kept = dest >= 0
    row_gate[dest[kept]] = g[kept]

    dx = np.zeros((T, d))
    y_rows = np.zeros((R, d))
    h = np.asarray(w1).shape[1]
    grads = {"dw1": np.zeros((E, h, d)), "dw2": np.zeros((E, d, h)),
             "dw3": np.zeros((E, h, d)) if w3 is not None else None,
             "db1": np.zeros((E, h)) if b1 is not None else None,
             "db2": np.zeros((E, d)) if b2 is not None else None}
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        if rows.size == 0:
            continue
        toks = row_token[rows]
        res = expert_ffn_backward(xs[toks], w1[e], w2[e], act, row_gate[rows, None] * dy[toks],
                                  None if w3 is None else w3[e], None if b1 is None else b1[e],
                                  None if b2 is None else b2[e])
        y_rows[rows] = res["y"]
        np.add.at(dx, toks, res["dx"])
        grads["dw1"][e] = res["dw1"]
        grads["dw2"][e] = res["dw2"]
        if w3 is not None:
            grads["dw3"][e] = res["dw3"]
        if b1 is not None:
            grads["db1"][e] = res["db1"]
        if b2 is not None:
            grads["db2"][e] = res["db2"]

    if ws1 is not None:
        S = np.asarray(ws1).shape[0]
        grads["dws1"] = np.zeros((S, h, d))
        grads["dws2"] = np.zeros((S, d, h))
        grads["dws3"] = np.zeros((S, h, d)) if ws3 is not None else None
        for s in range(S):
            res = expert_ffn_backward(xs, ws1[s], ws2[s], act, dy, None if ws3 is None else ws3[s])
            dx += res["dx"]
            grads["dws1"][s] = res["dw1"]
            grads["dws2"][s] = res["dw2"]
            if ws3 is not None:
                grads["dws3"][s] = res["dw3"]

    dg = np.zeros((T, k))
    for t in range(T):
        for s in range(k):
            if dest[t, s] >= 0:
                dg[t, s] = float(dy[t] @ y_rows[dest[t, s]])

    dH = np.zeros((T, E))
    np.put_along_axis(dH, idx, gate_softmax_backward(g, dg), axis=1)
    f = np.asarray(fwd["counts"], np.float64) / (T * k)
    if g_aux:
        dH += g_aux * aux_loss_logit_grad(H, f)
    if g_z:
        dH += g_z * z_loss_logit_grad(H)

    rb = router_backward(xs, w_g, dH, w_noise, eps)
    dx += rb["dx"]
    out = {"dx": dx, "dw_g": rb["dw_g"], "db_g": rb["db_g"] if b_g is not None else None,
           "dw_noise": rb["dw_noise"], "dg": dg, "dH": dH, "row_gate": row_gate,
           "y_rows": y_rows, "fwd": fwd}
    out.update(grads)
    return out


def softmax_backward(p, dS) -> np.ndarray:
    """Scores p = softmax(H) over all experts: dH[t,j] = p_tj (dS_tj - sum_i p_ti dS_ti)."""
    p = np.asarray(p, np.float64)
    dS = np.asarray(dS, np.float64)
    return p * (dS - (p * dS).sum(axis=1, keepdims=True))


def layer_loss_expert_choice(x, w_g, w1, w2, *, k: int, act: str, capacity_factor: float, dy,
                             g_aux: float = 0.0, g_z: float = 0.0, exact_logits: bool = True,
                             **kw) -> float:
    """B1's objective for the expert-choice forward (derivative checks)."""
    fwd = moe_forward_expert_choice(x, w_g, w1, w2, k=k, act=act,
                                    capacity_factor=capacity_factor,
                                    exact_logits=exact_logits, **kw)
    return (float(np.sum(np.asarray(dy, np.float64) * fwd["y"])) + g_aux * fwd["l_aux"]
            + g_z * z_loss(fwd["logits"]))


def moe_backward_expert_choice(x, w_g, w1, w2, *, k: int, act: str, capacity_factor: float, dy,
                               g_aux: float = 0.0, g_z: float = 0.0, w3=None, b_g=None,
                               w_noise=None, eps=None, b1=None, b2=None, ws1=None, ws3=None,
                               ws2=None, logits=None, exact_logits: bool = False) -> dict:
    """Gradients of L (B1) for expert-choice routing (EB1), in float64:
    every taken pair's row runs the expert backward with upstream S[t,e]*dy_t,
    dS[t,e] = dy_t . FFN_e(x_t), the logits get the full-softmax backward of
    dS plus the loss terms, then the router's parameters."""
    fwd = moe_forward_expert_choice(x, w_g, w1, w2, k=k, act=act,
                                    capacity_factor=capacity_factor, w3=w3, b_g=b_g,
                                    w_noise=w_noise, eps=eps, b1=b1, b2=b2, logits=logits,
                                    exact_logits=exact_logits)
    H = np.asarray(fwd["logits"], np.float64)
    S = np.asarray(fwd["scores"], np.float64)
    slot = np.asarray(fwd["slot"], np.int64)
    offsets = np.asarray(fwd["offsets"], np.int64)
    row_token = np.asarray(fwd["row_token"], np.int64)
    xs = np.asarray(x)
    T, d = xs.shape
    E = np.asarray(w_g).shape[0]
    dy = np.asarray(dy, np.float64)
    h = np.asarray(w1).shape[1]
    R = int(offsets[-1])
    row_gate = np.zeros(R)
    taken = slot >= 0
    row_gate[slot[taken]] = S[taken]

    dx = np.zeros((T, d))
    y_rows = np.zeros((R, d))
    grads = {"dw1": np.zeros((E, h, d)), "dw2": np.zeros((E, d, h)),
             "dw3": np.zeros((E, h, d)) if w3 is not None else None,
             "db1": np.zeros((E, h)) if b1 is not None else None,
             "db2": np.zeros((E, d)) if b2 is not None else None}
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        if rows.size == 0:
            continue
        toks = row_token[rows]
        res = expert_ffn_backward(xs[toks], w1[e], w2[e], act, row_gate[rows, None] * dy[toks],
                                  None if w3 is None else w3[e], None if b1 is None else b1[e],
                                  None if b2 is None else b2[e])
        y_rows[rows] = res["y"]
        np.add.at(dx, toks, res["dx"])
        for n in ("dw1", "dw2", "dw3", "db1", "db2"):
            if grads[n] is not None:
                grads[n][e] = res[n]
    if ws1 is not None:
        S_ = np.asarray(ws1).shape[0]
        grads["dws1"] = np.zeros((S_, h, d))
        grads["dws2"] = np.zeros((S_, d, h))
        grads["dws3"] = np.zeros((S_, h, d)) if ws3 is not None else None
        for s in range(S_):
            res = expert_ffn_backward(xs, ws1[s], ws2[s], act, dy, None if ws3 is None else ws3[s])
            dx += res["dx"]
            grads["dws1"][s] = res["dw1"]
            grads["dws2"][s] = res["dw2"]
            if ws3 is not None:
                grads["dws3"][s] = res["dw3"]

    dS = np.zeros((T, E))
    for t, e in zip(*np.nonzero(taken)):
        dS[t, e] = float(dy[t] @ y_rows[slot[t, e]])
    f = np.asarray(fwd["f"], np.float64)
    dH = softmax_backward(full_softmax(H), dS)
    if g_aux:
        dH += g_aux * aux_loss_logit_grad(H, f)
    if g_z:
        dH += g_z * z_loss_logit_grad(H)
    rb = router_backward(xs, w_g, dH, w_noise, eps)
    dx += rb["dx"]
    out = {"dx": dx, "dw_g": rb["dw_g"], "db_g": rb["db_g"] if b_g is not None else None,
           "dw_noise": rb["dw_noise"], "dS": dS, "dH": dH, "row_gate": row_gate,
           "y_rows": y_rows, "fwd": fwd}
    out.update(grads)
    return out
