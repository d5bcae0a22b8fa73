"""Pins of the oracle's overflow re-routing (CPU only).

"Mixture-of-experts Models", Level 2, "Overflow handling defines an output
contract": an assignment that finds its expert full may be re-routed to a
lower-ranked expert.  The page fixes no policy; the oracle's reading (RR1-RR4
in its header) is pinned by hand-worked cases, the page's capacity example and
invariants that any correct implementation of the reading satisfies.
"""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_reroute_hand_example():
    # C = 1, every token's first choice is expert 0.  Round 1: tokens 1 and 2
    # both propose expert 1 (their second choice), token 1 wins by arrival;
    # token 3 proposes expert 2 and gets it.  Round 2: token 2 tries expert 2,
    # full.  Round 3: token 2 has no fallback left and is dropped.
    H = np.array([[3, 2, 1], [3, 2, 1], [3, 2, 1], [3, 1, 2]], np.float32)
    r = O.dispatch_reroute(O.select_top_k(H, 1), H, 3, 1)
    assert r["final_expert"].ravel().tolist() == [0, 1, -1, 2]
    assert r["dest"].ravel().tolist() == [0, 1, -1, 2]
    assert r["row_token"].tolist() == [0, 1, 3]
    assert r["placed"].tolist() == [1, 1, 1] and r["counts"].tolist() == [4, 0, 0]
    assert r["rounds"] == 3


def test_reroute_on_the_capacity_worked_example():
    """The page's assignments [0,0,0,1,1,2,3,3] with capacity 2 overflow
    expert 0 once (flat index 2).  With token 2 ranking expert 2 second, the
    overflow lands on expert 2, which has one free slot: nothing is dropped."""
    g = json.load(open(os.path.join(GOLDEN, "capacity_worked_example.json")))
    a = np.array(g["assignments"])
    H = np.zeros((a.size, 4), np.float32)
    H[np.arange(a.size), a] = 2.0
    H[2, 2] = 1.0
    r = O.dispatch_reroute(a[:, None].astype(np.int32), H, 4, g["capacity"])
    assert r["final_expert"].ravel().tolist() == [0, 0, 2, 1, 1, 2, 3, 3]
    assert r["placed"].tolist() == [2, 2, 2, 2]
    # expert 2's rows: its primary token 5, then the re-routed token 2
    assert r["row_token"].tolist() == [0, 1, 3, 4, 5, 2, 6, 7]
    assert (r["dest"] >= 0).all()


def test_reroute_multiple_slots_take_distinct_fallbacks():
    # k = 2, E = 4, C = 1: tokens 0 and 1 both choose experts {0, 1}; token 1
    # loses both slots and they take its fallbacks 2 and 3 in one round
    H = np.array([[4, 3, 2, 1], [4, 3, 2, 1]], np.float32)
    r = O.dispatch_reroute(O.select_top_k(H, 2), H, 4, 1)
    assert r["final_expert"].tolist() == [[0, 1], [2, 3]]
    assert r["rounds"] == 1


def test_reroute_equals_drop_when_nothing_overflows():
    rng = np.random.default_rng(0)
    H = rng.standard_normal((50, 6)).astype(np.float32)
    idx = O.select_top_k(H, 2)
    C = int(np.bincount(idx.ravel(), minlength=6).max())
    r, d = O.dispatch_reroute(idx, H, 6, C), O.dispatch(idx, 6, C)
    for key in ("offsets", "dest", "row_token"):
        assert np.array_equal(r[key], d[key]), key
    assert r["rounds"] == 0


@pytest.mark.parametrize("seed", range(6))
def test_reroute_invariants(seed):
    rng = np.random.default_rng(seed)
    T, E, k = int(rng.integers(5, 80)), int(rng.integers(2, 9)), 1
    k = int(rng.integers(1, E)) if E > 1 else 1
    H = (rng.standard_normal((T, E)) + np.linspace(2, 0, E)).astype(np.float32)
    H[rng.random((T, E)) < 0.2] = 0.0  # ties
    idx = O.select_top_k(H, k)
    for C in (0, 1, max(1, T * k // (2 * E)), T * k // E, T):
        r = O.dispatch_reroute(idx, H, E, C)
        fe = r["final_expert"]
        assert (r["placed"] <= C).all()
        assert r["placed"].sum() == (fe >= 0).sum() == (r["dest"] >= 0).sum()
        rank = np.argsort(np.argsort(-H, axis=1, kind="stable"), axis=1)  # position of e
        for t in range(T):
            got = fe[t][fe[t] >= 0]
            assert len(set(got.tolist())) == got.size              # distinct experts
            for s in range(k):
                if fe[t, s] >= 0 and fe[t, s] != idx[t, s]:       # re-routed
                    assert fe[t, s] not in idx[t]
                    assert rank[t, fe[t, s]] >= k                   # ranked below the top k
        # rows: an expert's primary rows first, all rows of an expert contiguous
        for e in range(E):
            rows = r["row_token"][r["offsets"][e]:r["offsets"][e + 1]]
            assert ((fe == e).sum(axis=1)[rows] >= 1).all()
        # an assignment left unplaced means its token tried every fallback:
        # each was full when tried (loads never fall, so it ends full) or took
        # another slot of the same token
        F = O.fallback_order(H, k)
        for t, s in zip(*np.nonzero(fe < 0)):
            for e in F[t]:
                assert r["placed"][e] == C or e in fe[t]
