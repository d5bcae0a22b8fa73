"""CPU oracle for the forward pass of one sparse Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or call this module; the HIP
library never does, and nothing here is a fallback for it.

Plain NumPy/SciPy, float64 throughout (the pages fix no precision), written from
the pages' definitions so that a reader can check each step by eye.  Sources are
cited by page title and section:

  [MoE&SMS]  "Mixture-of-Experts & Sparse Model Scaling" (chipfoundryservices
             glossary): "Mathematical Formulation"; "Advanced Theory &
             Extensions"; appendix labs 1-3.
  [MoEM]     "Mixture-of-experts Models" (sempe.dev chapter): Level 2 "Router
             scores become a sparse dispatch decision", "Top-k selection has
             ties...", "Capacity limits make dispatch observable", "Overflow
             handling defines an output contract"; Level 3 imbalance example.
  [SMoE-arch] "Scaling Capacity via Sparse Mixture of Experts (MoE)
             Architectures" (quizzr): the router and layer snippets.
  [LLM-09]   "Large Language Models part 09: Sparse Mixture-of-Experts (MoE),
             Router, Switch" (shakilmahmud.com): section 2 (noisy top-k gating),
             section 3 (expert capacity), section 4 (auxiliary load balancing).
  [3D-lab]   "3D mixture-of-experts routing lab" (toy.new): Router and Capacity
             panels.

Readings taken where the pages are silent or disagree (each also listed in the
design notes):
  R1  Gates are the softmax over the k selected logits ([LLM-09] s.2), which is
      the same real number as the renormalised full-softmax probabilities of
      [MoE&SMS] lab 1 and [MoEM] Level 2.
  R2  Top-k order: logit descending, ties to the lower expert index, decided on
      the float32 logits; slot 0 is the best expert.
  R3  Capacity C = floor(factor * T * k / E) ([3D-lab] Capacity panel),
      evaluated in IEEE double left to right; dropless means C = T.
  R4  Drop priority is arrival order over the flat token-major assignment
      index t*k + s ([MoE&SMS] lab 3 generalised to k slots).  A dropped
      assignment contributes zero and the surviving gates are not renormalised.
  R5  f_i counts routed (pre-capacity) assignments / (T*k); P_i is the token
      mean of the FULL softmax of the logits ([MoE&SMS] lab 2); alpha = 1.
  R6  Noise: H = x W_g^T (+ b_g) + eps * softplus(x W_noise^T), eps supplied.
  R7  Shared experts take every token with weight 1, outside routing,
      capacity and the statistics ([MoE&SMS] "Advanced Theory & Extensions").
  R8  GELU is the exact erf form; SwiGLU is silu(x W1^T) * (x W3^T) then W2.

Expert-choice routing ([MoE&SMS] "Advanced Theory & Extensions": every expert
takes the tokens it scores highest, up to its capacity, so a token may be
processed by no expert or by several).  The page fixes neither the score nor
the tie rule; the readings:
  EC1 The score of token t for expert e is the softmax over experts of t's
      logits (the same probabilities P is built from), rounded once to
      float32; the ranking is decided on those float32 scores.
  EC2 Each expert takes C' = min(C, T) tokens, C = floor(factor * T * k / E)
      as in R3, k read as the average number of experts per token.
  EC3 Equal scores go to the lower token index.
  EC4 The gate of a (token, expert) pair is the token's float32 score for
      that expert, not renormalised over the experts that took the token.
  EC5 An expert's rows are laid out in ascending token order (layout only).
  EC6 f_i = rows of expert i / all rows (1/E here), P and L_aux as in R5, and
      the drop rate is the fraction of tokens that no expert took.

Overflow re-routing ([MoEM] Level 2 "Overflow handling defines an output
contract": an assignment that finds its expert full may be dropped, sent to a
lower-ranked expert, or kept on a residual path; [3D-lab] Capacity panel).
The pages fix no re-routing policy; the reading:
  RR1 A token's fallback experts are the ones ranked below its top k, in the
      same float32-logit order and tie rule; each is tried at most once.
  RR2 Rounds: every still-unplaced assignment proposes its token's next
      untried fallback (a token's unplaced slots, in slot order, take
      consecutive untried fallbacks); every expert accepts the proposals in
      arrival order up to its spare capacity C - load; the rest retry in the
      next round; an assignment whose token has no untried fallback left is
      dropped.
  RR3 A re-routed slot keeps its gate; only the expert that processes it
      changes.
  RR4 f_i still counts the router's (primary) assignments; the drop rate
      counts assignments left unplaced; an expert's rows are its primary
      kept assignments, then each round's accepted ones, in arrival order.

Router z-loss and routing diagnostics ([MoE&SMS] "Advanced Theory &
Extensions": a z-loss keeps router logits from growing large; "Benchmark
Datasets & Evaluation": utilisation histograms, routing entropy and the
fraction of tokens dropped; [MoEM] Level 3: overflow, imbalance measure).
The pages give no z-loss formula; the reading:
  Z1 z-loss = mean over tokens of (log sum_e exp H[t,e])^2, alpha = 1, on the
     float32 logits; routing entropy = mean over tokens of -sum_e p log p of
     the full softmax, in nats.

Layouts (row-major, every weight in out x in form, as an nn.Linear stores it):
  x [T,d]; w_g, w_noise [E,d]; b_g [E]; eps [T,E]; w1, w3 [E,h,d]; w2 [E,d,h];
  b1 [E,h]; b2 [E,d]; ws1, ws3 [S,h,d]; ws2 [S,d,h].
bfloat16 tensors arrive as uint16 bit patterns and are widened exactly.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf, expit

__all__ = [
    "to_f64", "softplus", "router_logits", "select_top_k", "selected_gates",
    "full_softmax", "capacity", "dispatch_in_arrival_order", "dispatch",
    "activation", "expert_ffn", "combine", "balance_stats", "moe_forward",
    "overflow_record", "expert_choice_scores", "expert_choice_select",
    "expert_choice_combine", "moe_forward_expert_choice", "routing_diagnostics",
    "fallback_order", "dispatch_reroute",
]


def to_f64(a) -> np.ndarray:
    """Exact widening: bfloat16 bit patterns (uint16) or float32 -> float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def softplus(z: np.ndarray) -> np.ndarray:
    """log(1 + e^z), in the overflow-free form max(z,0) + log1p(e^-|z|)."""
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def router_logits(x, w_g, b_g=None, w_noise=None, eps=None, rounded: bool = True) -> np.ndarray:
    """Router logits H [T,E], returned as float32.

    [MoE&SMS] "Mathematical Formulation": one logit per expert from a linear map
    of the token; [LLM-09] s.2: H_i = (x W_g)_i + eps * softplus((x W_noise)_i)
    with eps ~ N(0,1) supplied by the caller (R6).  An optional per-expert bias
    is added to the linear term ([SMoE-arch] router uses a biased linear layer).
    Computed in float64 and rounded once to float32: these float32 logits are
    what routing decides on (R2).  ``rounded=False`` returns the float64 value
    unrounded (derivative checks of the backward need a smooth map).
    """
    x64 = to_f64(x)
    H = x64 @ to_f64(w_g).T
    if b_g is not None:
        H = H + to_f64(b_g)[None, :]
    if w_noise is not None:
        if eps is None:
            raise ValueError("noisy gating needs eps")
        H = H + to_f64(eps) * softplus(x64 @ to_f64(w_noise).T)
    H32 = H.astype(np.float32)
    if not np.all(np.isfinite(H32)):
        raise FloatingPointError("non-finite router logits")
    return H32 if rounded else H


def select_top_k(H32: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per token, best first (R2).

    [MoE&SMS] "Mathematical Formulation" (TopK over the scores) and lab 1
    (descending order); [MoEM] Level 2 asks for a deterministic tie rule.
    A stable sort of the negated float32 logits orders by value descending
    and, among equal values (including -0.0 == +0.0), by lower index first.
    """
    H32 = np.asarray(H32, dtype=np.float32)
    E = H32.shape[1]
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    return np.argsort(-H32, axis=1, kind="stable")[:, :k].astype(np.int32)


def selected_gates(H32: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Gates [T,k]: softmax over the selected logits only (R1, [LLM-09] s.2).

    Shifted by the best selected logit (slot 0), as a softmax is computed
    stably; the k gates of a token sum to 1.
    """
    sel = np.take_along_axis(np.asarray(H32, np.float64), idx.astype(np.int64), axis=1)
    w = np.exp(sel - sel[:, :1])
    return w / w.sum(axis=1, keepdims=True)


def full_softmax(H32: np.ndarray) -> np.ndarray:
    """p_i = exp(g_i) / sum_j exp(g_j) over all E experts ([MoE&SMS]
    "Mathematical Formulation"), max-shifted as in its lab 1."""
    H = np.asarray(H32, np.float64)
    w = np.exp(H - H.max(axis=1, keepdims=True))
    return w / w.sum(axis=1, keepdims=True)


def capacity(capacity_factor: float, T: int, k: int, E: int) -> int:
    """Per-expert quota C = floor(factor * tokens * k / experts) ([3D-lab]
    Capacity panel; at k = 1 it is [LLM-09] s.3's factor * T / E).  A factor
    <= 0 means dropless: C = T, the most assignments one expert can receive
    because a token's k experts are distinct (R3)."""
    if capacity_factor <= 0:
        return int(T)
    return int(math.floor(capacity_factor * T * k / E))


def dispatch_in_arrival_order(idx: np.ndarray, E: int, C: int) -> dict:
    """Capacity check as a sequential walk over arrivals (R4).

    [MoE&SMS] lab 3: each arriving assignment is accepted while its expert's
    load is below capacity, otherwise dropped; generalised to k slots by
    walking the flat index t*k + s in increasing order.  Returns per-expert
    demand ``counts``, accepted ``kept``, and per assignment the position
    ``slot_rank`` it took in its expert's buffer, or -1 if dropped.
    """
    T, k = idx.shape
    load = [0] * E
    counts = [0] * E
    slot_rank = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for s in range(k):
            e = int(idx[t, s])
            counts[e] += 1
            if load[e] < C:
                slot_rank[t, s] = load[e]
                load[e] += 1
    return {"counts": np.array(counts, np.int64), "kept": np.array(load, np.int64),
            "slot_rank": slot_rank}


def dispatch(idx: np.ndarray, E: int, C: int) -> dict:
    """Dispatch tables for the expert-contiguous layout, vectorised.

    The rank of assignment (t,s) within its expert is the number of earlier
    flat assignments (t'*k+s' < t*k+s) to the same expert, which a stable sort
    of the flat expert ids yields; it is kept iff rank < C (same decisions as
    ``dispatch_in_arrival_order``).  [SMoE-arch] groups tokens by their expert;
    the buffers here hold, per expert, its kept assignments in arrival order:
      counts[e]   routed assignments (demand) of expert e
      kept[e]     min(counts[e], C)
      offsets     [E+1] exclusive prefix sum of kept
      dest[t,s]   row of the assignment in the expert-contiguous buffer, or -1
      row_token   [sum(kept)] the token held in each buffer row
    [MoEM] Level 2 capacity example: overflow = counts - kept.
    """
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    order = np.argsort(flat, kind="stable")
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    rank = np.empty_like(flat)
    rank[order] = np.arange(flat.size) - np.repeat(starts, counts)
    kept = np.minimum(counts, C)
    offsets = np.concatenate([[0], np.cumsum(kept)]).astype(np.int64)
    keep = rank < C
    dest = np.where(keep, offsets[flat] + rank, -1)
    row_token = np.empty(int(offsets[-1]), dtype=np.int64)
    tok = np.arange(flat.size) // k
    row_token[dest[keep]] = tok[keep]
    return {"counts": counts, "kept": kept, "offsets": offsets,
            "dest": dest.reshape(T, k), "row_token": row_token,
            "rank": rank.reshape(T, k), "capacity": int(C)}


def activation(act: str, a: np.ndarray, b: np.ndarray | None = None) -> np.ndarray:
    """Expert non-linearities (R8): exact GELU 0.5 a (1 + erf(a / sqrt 2));
    ReLU max(a, 0); SwiGLU silu(a) * b with silu(a) = a * sigmoid(a)."""
    if act == "gelu":
        return 0.5 * a * (1.0 + erf(a / math.sqrt(2.0)))
    if act == "relu":
        return np.maximum(a, 0.0)
    if act == "swiglu":
        if b is None:
            raise ValueError("swiglu needs the up projection")
        return a * expit(a) * b
    raise ValueError(act)


def expert_ffn(x_rows, w1, w2, act, w3=None, b1=None, b2=None) -> np.ndarray:
    """One expert FFN on a set of token rows, float64.

    [MoE&SMS] "Core Concepts": an expert has the architecture of the dense FFN
    it replaces with its own weights; lab 4 counts one hidden layer with
    biases.  y = act(x W1^T (+ b1) [, x W3^T]) W2^T (+ b2); the hidden layer is
    kept unrounded.
    """
    x = to_f64(x_rows)
    a = x @ to_f64(w1).T
    if b1 is not None:
        a = a + to_f64(b1)[None, :]
    u = x @ to_f64(w3).T if w3 is not None else None
    hid = activation(act, a, u)
    y = hid @ to_f64(w2).T
    if b2 is not None:
        y = y + to_f64(b2)[None, :]
    return y


def combine(T, d, idx, gates, dest, expert_rows_out, tokens, shared_out=None) -> np.ndarray:
    """y_t = shared_t + sum over the token's slots s of [kept] g_ts * E_e(x_t).

    [MoE&SMS] "Mathematical Formulation": the weighted sum runs over the
    selected experts only; [LLM-09] s.1 writes it as sum_i G(x)_i E_i(x).
    A dropped slot adds nothing and the other gates are not rescaled (R4,
    [MoEM] "Overflow handling defines an output contract").  Shared experts
    add with weight 1 (R7).  ``expert_rows_out`` maps a buffer row to that
    assignment's expert output.
    """
    y = np.zeros((len(tokens), d), np.float64)
    if shared_out is not None:
        y += shared_out
    k = idx.shape[1]
    for j, t in enumerate(tokens):
        for s in range(k):
            r = int(dest[t, s])
            if r >= 0:
                y[j] += gates[t, s] * expert_rows_out[r]
    return y


def balance_stats(counts, kept, P, T: int, k: int, E: int) -> dict:
    """Switch load-balance statistics (R5).

    [MoE&SMS] "Mathematical Formulation": L_aux = N * sum_i f_i P_i, f_i the
    hard fraction of assignments routed to expert i, P_i the mean router
    probability; [LLM-09] s.4 gives the same with alpha (taken as 1).
    Diagnostics from [MoEM]: overflow per expert, drop rate (lab 3 of
    [MoE&SMS]: 1 - fraction processed), load coefficient of variation and the
    absolute deviation from equal load (Level 3 example).
    """
    counts = np.asarray(counts, np.float64)
    kept = np.asarray(kept, np.float64)
    f = counts / (T * k)
    l_aux = E * float(np.sum(f * P))
    mean = counts.mean()
    return {
        "f": f, "P": P, "l_aux": l_aux,
        "drop_rate": 1.0 - kept.sum() / (T * k),
        "overflow": counts - kept,
        "load_cv": float(counts.std() / mean) if mean > 0 else 0.0,
        "deviation": float(np.abs(counts - T * k / E).sum()),
    }


def moe_forward(x, w_g, w1, w2, *, k: int, act: str, capacity_factor: float,
                w3=None, b_g=None, w_noise=None, eps=None, b1=None, b2=None,
                ws1=None, ws3=None, ws2=None, logits=None, tokens=None,
                overflow: str = "drop", exact_logits: bool = False) -> dict:
    """The whole layer forward, step by step.

    1. router logits H (or the supplied float32 ``logits``);
    2. top-k experts and their gates, full softmax for P;
    3. counts, capacity and drops in arrival order, expert-contiguous tables;
    4. every expert on its kept rows (restricted to ``tokens`` if given);
    5. gate-weighted combine back to token order, plus shared experts, and
       the load-balance statistics.
    ``tokens`` (default all) selects which output rows to compute; steps 1-3
    and the statistics always cover the whole batch, since capacity couples
    tokens through their arrival order ([MoEM] "Routing is conditional on a
    token and its batch context").  ``overflow="reroute"`` sends assignments
    that find their expert full to lower-ranked experts (RR1-RR4) instead of
    dropping them.  ``exact_logits`` keeps the logits in float64 instead of
    rounding them to float32 (for derivative checks; the top-k order is still
    decided in float32).
    """
    T, d = np.asarray(x).shape
    E = np.asarray(w_g).shape[0]
    if logits is None:
        H = router_logits(x, w_g, b_g, w_noise, eps, rounded=not exact_logits)
    else:
        H = np.asarray(logits, np.float64 if exact_logits else np.float32)
    idx = select_top_k(H, k)
    g = selected_gates(H, idx)
    P = full_softmax(H).mean(axis=0)
    C = capacity(capacity_factor, T, k, E)
    disp = dispatch_reroute(idx, H, E, min(C, T)) if overflow == "reroute" else dispatch(idx, E, C)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    want = np.zeros(T, bool)
    want[tokens] = True

    rows_out = {}
    offsets, row_token = disp["offsets"], disp["row_token"]
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        rows = rows[want[row_token[rows]]]
        if rows.size == 0:
            continue
        ye = expert_ffn(np.asarray(x)[row_token[rows]], w1[e], w2[e], act,
                        None if w3 is None else w3[e],
                        None if b1 is None else b1[e], None if b2 is None else b2[e])
        for r, v in zip(rows, ye):
            rows_out[int(r)] = v

    shared = None
    if ws1 is not None:
        shared = np.zeros((len(tokens), d), np.float64)
        for s in range(ws1.shape[0]):
            shared += expert_ffn(np.asarray(x)[tokens], ws1[s], ws2[s], act,
                                 None if ws3 is None else ws3[s])
    y = combine(T, d, idx, g, disp["dest"], rows_out, tokens, shared)
    stats = balance_stats(disp["counts"], disp["kept"], P, T, k, E)
    if overflow == "reroute":  # RR4: what is left unplaced after re-routing
        stats["drop_rate"] = float(np.mean(np.asarray(disp["dest"]) < 0)) if T else 0.0
    return {"logits": H, "idx": idx, "gates": g, "prob_mean": P, "capacity": C,
            **disp, **stats, "y": y, "tokens": tokens, "shared": shared}


def overflow_record(idx: np.ndarray, dest: np.ndarray) -> list:
    """Per affected token: selected experts, successful assignments, fallback
    type and final path ([MoEM] "Overflow handling defines an output
    contract").  The fallback here is always "drop"."""
    rec = []
    for t in range(idx.shape[0]):
        lost = [int(e) for e, r in zip(idx[t], dest[t]) if r < 0]
        if lost:
            rec.append({"token": t, "selected": [int(e) for e in idx[t]],
                        "processed": [int(e) for e, r in zip(idx[t], dest[t]) if r >= 0],
                        "fallback": "drop", "dropped": lost})
    return rec


def expert_choice_scores(H32: np.ndarray) -> np.ndarray:
    """Scores for expert-choice routing (EC1): the per-token softmax over the
    experts, computed in float64 from the float32 logits, rounded to float32."""
    return full_softmax(H32).astype(np.float32)


def expert_choice_select(S32: np.ndarray, C: int) -> dict:
    """Every expert takes the min(C, T) tokens with the highest float32 score,
    equal scores to the lower token index (EC2, EC3): a stable sort of the
    negated column.  Rows are expert-contiguous, each expert's tokens in
    ascending order (EC5).  ``slot[t, e]`` is the row holding (t, e), or -1."""
    S32 = np.asarray(S32, np.float32)
    T, E = S32.shape
    Cp = min(int(C), T)
    row_token = np.empty(E * Cp, np.int32)
    slot = np.full((T, E), -1, np.int32)
    for e in range(E):
        chosen = np.sort(np.argsort(-S32[:, e], kind="stable")[:Cp])
        row_token[e * Cp:(e + 1) * Cp] = chosen
        slot[chosen, e] = e * Cp + np.arange(Cp, dtype=np.int32)
    counts = np.full(E, Cp, np.int64)
    offsets = np.arange(E + 1, dtype=np.int64) * Cp
    return {"counts": counts, "offsets": offsets, "row_token": row_token, "slot": slot,
            "capacity_used": Cp}


def expert_choice_combine(d, S32, slot, rows_out, tokens, shared_out=None) -> np.ndarray:
    """y_t = shared experts + sum over e in ascending order of the experts that
    took t of S[t, e] * FFN_e(x_t), in float64 (EC4); a token no expert took
    gets the shared part only."""
    y = np.zeros((len(tokens), d), np.float64) if shared_out is None else np.array(shared_out, np.float64)
    for i, t in enumerate(tokens):
        for e in range(slot.shape[1]):
            r = int(slot[t, e])
            if r >= 0:
                y[i] += np.float64(S32[t, e]) * rows_out[r]
    return y


def moe_forward_expert_choice(x, w_g, w1, w2, *, k: int, act: str, capacity_factor: float,
                              w3=None, b_g=None, w_noise=None, eps=None, b1=None, b2=None,
                              ws1=None, ws3=None, ws2=None, logits=None, scores=None,
                              tokens=None, exact_logits: bool = False) -> dict:
    """The layer forward with expert-choice routing.

    1. router logits H (or the supplied float32 ``logits``);
    2. scores S (EC1, or the supplied float32 ``scores``), P from H as in R5;
    3. every expert takes its min(C, T) best tokens (EC2, EC3);
    4. every expert on its rows (restricted to ``tokens`` if given);
    5. y_t = shared experts + the sum over the experts that took t, in expert
       order, of S[t, e] * FFN_e(x_t) (EC4); statistics (EC6).
    ``exact_logits`` keeps H and S in float64, unrounded (derivative checks;
    the selection is still decided on float32 scores).
    """
    T, d = np.asarray(x).shape
    E = np.asarray(w_g).shape[0]
    if exact_logits:
        H = (router_logits(x, w_g, b_g, w_noise, eps, rounded=False) if logits is None
             else np.asarray(logits, np.float64))
        S = full_softmax(H) if scores is None else np.asarray(scores, np.float64)
    else:
        H = router_logits(x, w_g, b_g, w_noise, eps) if logits is None else np.asarray(logits, np.float32)
        S = expert_choice_scores(H) if scores is None else np.asarray(scores, np.float32)
    P = full_softmax(H).mean(axis=0)
    C = capacity(capacity_factor, T, k, E)
    sel = expert_choice_select(S, C)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    want = np.zeros(T, bool)
    want[tokens] = True

    xs = np.asarray(x)
    rows_out = {}
    for e in range(E):
        rows = np.arange(sel["offsets"][e], sel["offsets"][e + 1])
        rows = rows[want[sel["row_token"][rows]]]
        if rows.size == 0:
            continue
        ye = expert_ffn(xs[sel["row_token"][rows]], w1[e], w2[e], act, None if w3 is None else w3[e],
                        None if b1 is None else b1[e], None if b2 is None else b2[e])
        for r, v in zip(rows, ye):
            rows_out[int(r)] = v
    shared = None
    if ws1 is not None:
        shared = np.zeros((len(tokens), d), np.float64)
        for s_ in range(ws1.shape[0]):
            shared += expert_ffn(xs[tokens], ws1[s_], ws2[s_], act, None if ws3 is None else ws3[s_])
    y = expert_choice_combine(d, S, sel["slot"], rows_out, tokens, shared)
    counts = sel["counts"]
    f = counts / max(1, counts.sum())
    covered = (sel["slot"] >= 0).any(axis=1)
    return {"logits": H, "scores": S, "prob_mean": P, "capacity": C, **sel, "f": f, "P": P,
            "l_aux": float(E * np.sum(f * P)), "drop_rate": float(1.0 - covered.mean()) if T else 0.0,
            "experts_per_token": (sel["slot"] >= 0).sum(axis=1), "y": y, "tokens": tokens,
            "shared": shared}


def routing_diagnostics(H32, counts, kept, dest, C: int, T: int, k: int, E: int) -> dict:
    """Router z-loss (Z1) and routing diagnostics of one token-choice batch:
    routing entropy, imbalance (load CV, absolute deviation from the equal
    share, peak-to-mean load), overflow per expert, utilisation kept / C, and
    the fractions of tokens that lost all or some of their k assignments."""
    H = np.asarray(H32, np.float64)
    m = H.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(H - m).sum(axis=1, keepdims=True)))[:, 0]
    p = full_softmax(H32)
    ent = lse - (p * H).sum(axis=1)  # -sum p log p with log p = H - lse
    counts = np.asarray(counts, np.float64)
    kept = np.asarray(kept, np.float64)
    lost = (np.asarray(dest) < 0).sum(axis=1)
    mean = counts.mean()
    return {
        "z_loss": float(np.mean(lse ** 2)),
        "entropy": float(np.mean(ent)),
        "load_cv": float(counts.std() / mean) if mean > 0 else 0.0,
        "deviation": float(np.abs(counts - T * k / E).sum()),
        "peak_to_mean": float(counts.max() / mean) if mean > 0 else 0.0,
        "overflow": counts - kept,
        "overflow_total": float((counts - kept).sum()),
        "utilisation": kept / C if C > 0 else np.zeros(E),
        "tokens_fully_dropped": float(np.mean(lost == k)),
        "tokens_partly_dropped": float(np.mean((lost > 0) & (lost < k))),
    }


def fallback_order(H32: np.ndarray, k: int) -> np.ndarray:
    """[T, E-k]: each token's experts ranked k+1-th and below (RR1)."""
    return np.argsort(-np.asarray(H32, np.float32), axis=1, kind="stable")[:, k:].astype(np.int32)


def dispatch_reroute(idx: np.ndarray, H32: np.ndarray, E: int, C: int) -> dict:
    """Capacity with overflow re-routing (RR1-RR4): the arrival-order pass of
    ``dispatch`` first, then rounds of fallback proposals.  Returns the same
    tables as ``dispatch`` (offsets, dest and row_token over the final
    placement; counts are the primary ones) plus ``final_expert`` [T,k] (-1
    when dropped), ``placed`` per expert and ``rounds``."""
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    prim = dispatch(idx, E, C)
    load = np.asarray(prim["kept"], np.int64).copy()
    flat_dest = prim["dest"].reshape(-1)
    final_e = np.where(flat_dest >= 0, idx.reshape(-1), -1)
    row_in_e = np.where(flat_dest >= 0, prim["rank"].reshape(-1), -1)
    F = fallback_order(H32, k)
    nf = E - k
    ptr = np.zeros(T, np.int64)
    unplaced = [i for i in range(T * k) if flat_dest[i] < 0]
    rounds = 0
    while unplaced:
        rounds += 1
        proposals = []
        seen = {}
        for i in unplaced:                     # consecutive untried fallbacks per token
            t = i // k
            j = seen.get(t, 0)
            seen[t] = j + 1
            q = ptr[t] + j
            proposals.append(int(F[t, q]) if q < nf else -1)
        for t, n in seen.items():
            ptr[t] += n
        taken = np.zeros(E, np.int64)
        still = []
        for i, e in zip(unplaced, proposals):  # arrival order
            if e < 0:
                continue                        # no fallback left: dropped
            if load[e] + taken[e] < C:
                final_e[i] = e
                row_in_e[i] = load[e] + taken[e]
                taken[e] += 1
            else:
                still.append(i)
        load += taken
        unplaced = still
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(load)
    dest = np.where(final_e >= 0, offsets[np.maximum(final_e, 0)] + row_in_e, -1)
    row_token = np.full(int(offsets[-1]), -1, np.int64)
    ok = dest >= 0
    row_token[dest[ok]] = np.arange(T * k)[ok] // k
    return {"counts": prim["counts"], "kept": prim["kept"], "placed": load, "offsets": offsets,
            "dest": dest.reshape(T, k), "row_token": row_token,
            "final_expert": final_e.reshape(T, k), "rounds": rounds}
