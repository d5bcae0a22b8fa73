"""Plants plausible mistakes in the CPU oracle and checks the pins catch each.

Every mutation replaces one oracle function (in the oracle module and in the
package namespace the pin tests use) with a subtly wrong variant: a dropped
term, a wrong sign or index, a transposed reading, a different rounding.  The
pin suite must fail for every one of them.  Runs on the CPU only.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
import oracle.moe_oracle as M
import tests.test_oracle_expert_choice as ecpins
import tests.test_oracle_pins as pins
import tests.test_oracle_reroute as rrpins

ORIG = {n: getattr(M, n) for n in M.__all__}


def _router_no_bias(x, w_g, b_g=None, w_noise=None, eps=None):
    return ORIG["router_logits"](x, w_g, None, w_noise, eps)


def _router_linear_noise(x, w_g, b_g=None, w_noise=None, eps=None):
    H = M.to_f64(x) @ M.to_f64(w_g).T
    if b_g is not None:
        H = H + M.to_f64(b_g)
    if w_noise is not None:
        H = H + M.to_f64(eps) * (M.to_f64(x) @ M.to_f64(w_noise).T)
    return H.astype(np.float32)


def _router_noise_sign(x, w_g, b_g=None, w_noise=None, eps=None):
    return ORIG["router_logits"](x, w_g, b_g, w_noise, None if eps is None else -eps)


def _topk_ties_high(H32, k):
    H32 = np.asarray(H32, np.float32)
    E = H32.shape[1]
    return (E - 1 - np.argsort(-H32[:, ::-1], axis=1, kind="stable")[:, :k]).astype(np.int32)


def _topk_ascending(H32, k):
    return np.argsort(np.asarray(H32, np.float32), axis=1, kind="stable")[:, :k].astype(np.int32)


def _gates_unnormalised(H32, idx):
    return np.take_along_axis(M.full_softmax(H32), idx.astype(np.int64), axis=1)


def _capacity_round(cf, T, k, E):
    return int(T) if cf <= 0 else int(round(cf * T * k / E))


def _capacity_no_k(cf, T, k, E):
    return int(T) if cf <= 0 else int(math.floor(cf * T / E))


def _dispatch_slot_major(idx, E, C):
    T, k = idx.shape
    d = ORIG["dispatch"](idx.T.copy(), E, C)  # arrival order s*T + t
    d["dest"] = d["dest"].T.copy()
    d["rank"] = d["rank"].T.copy()
    return d


def _dispatch_off_by_one(idx, E, C):
    return ORIG["dispatch"](idx, E, C + 1)


def _combine_renormalised(T, d, idx, gates, dest, rows_out, tokens, shared_out=None):
    kept = dest >= 0
    g = gates * kept
    s = g.sum(1, keepdims=True)
    g = np.divide(g, s, out=np.zeros_like(g), where=s > 0)
    return ORIG["combine"](T, d, idx, g, dest, rows_out, tokens, shared_out)


def _ffn_no_b2(x_rows, w1, w2, act, w3=None, b1=None, b2=None):
    return ORIG["expert_ffn"](x_rows, w1, w2, act, w3, b1, None)


def _act_swapped_or_tanh(act, a, b=None):
    if act == "swiglu":
        return b * expit(b) * a
    if act == "gelu":
        return 0.5 * a * (1 + np.tanh(math.sqrt(2 / math.pi) * (a + 0.044715 * a ** 3)))
    return ORIG["activation"](act, a, b)


def _stats_f_swapped(counts, kept, P, T, k, E):
    return ORIG["balance_stats"](np.asarray(counts)[::-1], kept, P, T, k, E)


def _stats_f_over_T(counts, kept, P, T, k, E):
    return ORIG["balance_stats"](np.asarray(counts) * k, kept, P, T, k, E)


def _forward_sparse_P(*a, **kw):
    out = ORIG["moe_forward"](*a, **kw)
    T = out["idx"].shape[0]
    sparse = np.zeros((T, out["prob_mean"].size))
    np.put_along_axis(sparse, out["idx"].astype(np.int64), out["gates"], 1)
    out["prob_mean"] = sparse.mean(0)
    return out


def _ec_ties_high(S32, C):
    S32 = np.asarray(S32, np.float32)
    T = S32.shape[0]
    out = ORIG["expert_choice_select"](S32[::-1].copy(), C)
    Cp = out["capacity_used"]
    E = S32.shape[1]
    rt = (T - 1 - out["row_token"]).reshape(E, Cp) if Cp else out["row_token"].reshape(E, 0)
    rt = np.sort(rt, axis=1).reshape(-1).astype(np.int32)
    slot = np.full((T, E), -1, np.int32)
    for e in range(E):
        slot[rt[e * Cp:(e + 1) * Cp], e] = e * Cp + np.arange(Cp)
    out.update(row_token=rt, slot=slot)
    return out


def _ec_softmax_over_tokens(H32):
    H = np.asarray(H32, np.float64)
    w = np.exp(H - H.max(axis=0, keepdims=True))
    return (w / w.sum(axis=0, keepdims=True)).astype(np.float32)


def _ec_combine_renormalised(d, S32, slot, rows_out, tokens, shared_out=None):
    took = slot >= 0
    S = np.asarray(S32, np.float64) * took
    tot = S.sum(1, keepdims=True)
    S = np.divide(S, tot, out=np.zeros_like(S), where=tot > 0)
    return ORIG["expert_choice_combine"](d, S, slot, rows_out, tokens, shared_out)


def _ec_no_clip(S32, C):
    S32 = np.asarray(S32, np.float32)
    T, E = S32.shape
    row_token = np.empty(E * C, np.int32)
    slot = np.full((T, E), -1, np.int32)
    for e in range(E):
        chosen = np.sort(np.argsort(-S32[:, e], kind="stable")[:C])
        row_token[e * C:(e + 1) * C] = chosen
        slot[chosen, e] = e * C + np.arange(C)
    return {"counts": np.full(E, C), "offsets": np.arange(E + 1) * C, "row_token": row_token,
            "slot": slot, "capacity_used": C}


def _ec_rows_in_score_order(S32, C):
    out = ORIG["expert_choice_select"](S32, C)
    S32 = np.asarray(S32, np.float32)
    T, E = S32.shape
    Cp = out["capacity_used"]
    rt = out["row_token"].copy()
    for e in range(E):
        seg = rt[e * Cp:(e + 1) * Cp]
        rt[e * Cp:(e + 1) * Cp] = seg[np.argsort(-S32[seg, e], kind="stable")]
        out["slot"][rt[e * Cp:(e + 1) * Cp], e] = e * Cp + np.arange(Cp)
    out["row_token"] = rt
    return out


def _diag_z_unsquared(H32, counts, kept, dest, C, T, k, E):
    d = ORIG["routing_diagnostics"](H32, counts, kept, dest, C, T, k, E)
    H = np.asarray(H32, np.float64)
    m = H.max(axis=1, keepdims=True)
    d["z_loss"] = float(np.mean(m[:, 0] + np.log(np.exp(H - m).sum(axis=1))))
    return d


def _diag_entropy_bits(H32, counts, kept, dest, C, T, k, E):
    d = ORIG["routing_diagnostics"](H32, counts, kept, dest, C, T, k, E)
    d["entropy"] = d["entropy"] / math.log(2.0)
    return d


def _diag_any_loss_is_full(H32, counts, kept, dest, C, T, k, E):
    d = ORIG["routing_diagnostics"](H32, counts, kept, dest, C, T, k, E)
    lost = (np.asarray(dest) < 0).sum(axis=1)
    d["tokens_fully_dropped"] = float(np.mean(lost > 0))
    return d


def _stats_cv_sample_std(counts, kept, P, T, k, E):
    st = ORIG["balance_stats"](counts, kept, P, T, k, E)
    c = np.asarray(counts, np.float64)
    st["load_cv"] = float(c.std(ddof=1) / c.mean()) if c.mean() > 0 else 0.0
    return st


def _diag_cv_sample_std(H32, counts, kept, dest, C, T, k, E):
    d = ORIG["routing_diagnostics"](H32, counts, kept, dest, C, T, k, E)
    c = np.asarray(counts, np.float64)
    d["load_cv"] = float(c.std(ddof=1) / c.mean()) if c.mean() > 0 else 0.0
    return d


def _rr_fallback_reversed(H32, k):
    return ORIG["fallback_order"](H32, k)[:, ::-1].copy()


def _rr_variant(idx, H32, E, C, retry=True, reverse_arrival=False, reroute_first=False):
    """The re-routing rounds with one planted change."""
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    prim = M.dispatch(idx, E, C)
    load = np.asarray(prim["kept"], np.int64).copy()
    fd = prim["dest"].reshape(-1)
    fe = np.where(fd >= 0, idx.reshape(-1), -1)
    rin = np.where(fd >= 0, prim["rank"].reshape(-1), -1)
    F = M.fallback_order(H32, k)
    ptr = np.zeros(T, np.int64)
    un = [i for i in range(T * k) if fd[i] < 0]
    rerouted = np.zeros(T * k, bool)
    rounds = 0
    while un:
        rounds += 1
        props, seen = [], {}
        for i in un:
            t = i // k
            j = seen.get(t, 0)
            seen[t] = j + 1
            q = ptr[t] + j
            props.append(int(F[t, q]) if q < E - k else -1)
        for t, n in seen.items():
            ptr[t] += n
        taken = np.zeros(E, np.int64)
        still = []
        order = list(zip(un, props))
        if reverse_arrival:
            order = order[::-1]
        for i, e in order:
            if e < 0:
                continue
            if load[e] + taken[e] < C:
                fe[i], rin[i] = e, load[e] + taken[e]
                taken[e] += 1
                rerouted[i] = True
            elif retry:
                still.append(i)
        load += taken
        un = sorted(still)
    if reroute_first:  # re-routed rows before the primary ones
        for e in range(E):
            mine = np.nonzero(fe == e)[0]
            rr = [i for i in mine if rerouted[i]]
            pr = [i for i in mine if not rerouted[i]]
            for pos, i in enumerate(rr + pr):
                rin[i] = pos
    off = np.zeros(E + 1, np.int64)
    off[1:] = np.cumsum(load)
    dest = np.where(fe >= 0, off[np.maximum(fe, 0)] + rin, -1)
    rt = np.full(int(off[-1]), -1, np.int64)
    ok = dest >= 0
    rt[dest[ok]] = np.arange(T * k)[ok] // k
    return {"counts": prim["counts"], "kept": prim["kept"], "placed": load, "offsets": off,
            "dest": dest.reshape(T, k), "row_token": rt, "final_expert": fe.reshape(T, k),
            "rounds": rounds}


MUTATIONS = {
    "router drops the bias": ("router_logits", _router_no_bias),
    "noise without softplus": ("router_logits", _router_linear_noise),
    "noise sign flipped": ("router_logits", _router_noise_sign),
    "ties go to the higher index": ("select_top_k", _topk_ties_high),
    "top-k picks the smallest": ("select_top_k", _topk_ascending),
    "gates not renormalised": ("selected_gates", _gates_unnormalised),
    "capacity rounded, not floored": ("capacity", _capacity_round),
    "capacity without k": ("capacity", _capacity_no_k),
    "slot-major drop priority": ("dispatch", _dispatch_slot_major),
    "capacity off by one": ("dispatch", _dispatch_off_by_one),
    "surviving gates rescaled": ("combine", _combine_renormalised),
    "second bias dropped": ("expert_ffn", _ffn_no_b2),
    "swiglu halves swapped / tanh gelu": ("activation", _act_swapped_or_tanh),
    "f indices reversed": ("balance_stats", _stats_f_swapped),
    "f divided by T, not T*k": ("balance_stats", _stats_f_over_T),
    "P from the sparse gates": ("moe_forward", _forward_sparse_P),
    "expert choice: ties to the higher token": ("expert_choice_select", _ec_ties_high),
    "expert choice: softmax over tokens": ("expert_choice_scores", _ec_softmax_over_tokens),
    "expert choice: gates renormalised": ("expert_choice_combine", _ec_combine_renormalised),
    "expert choice: capacity not clipped at T": ("expert_choice_select", _ec_no_clip),
    "expert choice: rows in score order": ("expert_choice_select", _ec_rows_in_score_order),
    "z-loss not squared": ("routing_diagnostics", _diag_z_unsquared),
    "entropy in bits": ("routing_diagnostics", _diag_entropy_bits),
    "a partial drop counted as a full one": ("routing_diagnostics", _diag_any_loss_is_full),
    "load CV from the sample std (statistics)": ("balance_stats", _stats_cv_sample_std),
    "load CV from the sample std (diagnostics)": ("routing_diagnostics", _diag_cv_sample_std),
    "re-route: fallbacks from the lowest rank": ("fallback_order", _rr_fallback_reversed),
    "re-route: no retry after a rejection": ("dispatch_reroute", lambda *a: _rr_variant(*a, retry=False)),
    "re-route: later arrivals win": ("dispatch_reroute", lambda *a: _rr_variant(*a, reverse_arrival=True)),
    "re-route: re-routed rows first": ("dispatch_reroute", lambda *a: _rr_variant(*a, reroute_first=True)),
}

PIN_TESTS = [
    pins.test_top2_worked_example,
    pins.test_capacity_worked_example,
    pins.test_load_deviation_example,
    pins.test_load_cv_hand_worked_values,
    pins.test_topk_brute_force_with_ties_and_signed_zero,
    pins.test_gate_closed_forms,
    pins.test_router_identity_rows_give_weight_columns,
    pins.test_router_noise_reduces_and_matches_softplus,
    pins.test_capacity_formula_values,
    lambda: pins.test_dispatch_brute_force(3, 3, 2),
    lambda: [pins.test_dense_equivalence_E1_k1(a) for a in ("gelu", "relu", "swiglu")],
    pins.test_identical_experts_and_drops,
    pins.test_laux_closed_forms,
    pins.test_activations_match_library_forms,
    ecpins.test_ec_hand_example,
    ecpins.test_ec_ranks_on_scores_not_logits,
    ecpins.test_ec_uniform_scores_take_lowest_indices,
    lambda: ecpins.test_ec_brute_force_with_ties(3, 2),
    ecpins.test_ec_every_expert_full_and_stats,
    ecpins.test_ec_full_capacity_identical_experts_is_the_dense_ffn,
    ecpins.test_ec_single_expert_is_exactly_dense,
    ecpins.test_ec_partial_coverage_gates_are_raw_scores,
    ecpins.test_ec_capacity_above_batch_and_zero,
    pins.test_zloss_and_entropy_closed_forms,
    pins.test_diagnostics_on_the_capacity_worked_example,
    pins.test_diagnostics_partial_drops_with_two_slots,
    rrpins.test_reroute_hand_example,
    rrpins.test_reroute_on_the_capacity_worked_example,
    rrpins.test_reroute_multiple_slots_take_distinct_fallbacks,
    rrpins.test_reroute_equals_drop_when_nothing_overflows,
    lambda: [rrpins.test_reroute_invariants(s_) for s_ in range(3)],
]


def _sequential_reference_ok():
    """The sequential arrival walk is the definition; a mutated vectorised
    dispatch must disagree with it somewhere on the tiny-batch grid."""
    for idx in pins._all_idx_patterns(3, 3, 2):
        for cf in (0.5, 1.0, 1.5):
            C = ORIG["capacity"](cf, 3, 2, 3)
            seq = ORIG["dispatch_in_arrival_order"](idx, 3, C)
            vec = M.dispatch(idx, 3, C)
            if not np.array_equal(seq["kept"], vec["kept"]):
                return False
            if not np.array_equal(seq["slot_rank"] >= 0, vec["dest"] >= 0):
                return False
    return True


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    fn_name, bad = MUTATIONS[name]
    monkeypatch.setattr(M, fn_name, bad)
    monkeypatch.setattr(oracle, fn_name, bad)
    caught = []
    for t in PIN_TESTS:
        try:
            t()
        except Exception:  # an assertion or an error: the pin fired
            caught.append(t)
    if fn_name == "dispatch" and not _sequential_reference_ok():
        caught.append("sequential walk")
    assert caught, f"no pin caught the planted mistake: {name}"


def test_unmutated_oracle_passes_every_pin():
    for t in PIN_TESTS:
        t()
    assert _sequential_reference_ok()
