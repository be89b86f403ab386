"""Pins of the planner oracle against what the pages and the mathematics fix.

* hand-worked plans of the stated rule (tests/golden/plan_examples.json);
* exhaustive enumeration of every routing at tiny shapes, each plan checked by
  an invariant checker that does not know the rule (exactly S*K per rank, a
  bijection, slots served by their expert, one remote group per rank, B rules);
* special cases with a textbook answer: one rank (a stable counting sort),
  perfectly balanced routing (no replicas), one hot group (a star);
* the slot rank t against its literal definition;
* the checker itself rejects planted mistakes.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import plan as P
from oracle.check import check_plan, check_order

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_examples.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked_plans(case):
    c = case
    topk = np.array(c["topk_idx"], dtype=np.int32)
    pl = P.plan(topk, c["R"], c["S"], c["E"], c["K"], c["B"], c["mode"])
    assert pl.T.tolist() == c["T"]
    assert pl.parent == c["parent"]
    assert [[list(g) for g in gl] for gl in pl.gifts] == c["gifts"]
    assert pl.cu_seqlens.tolist() == c["cu_seqlens"]
    assert pl.replica_expert.tolist() == c["replica_expert"]
    assert pl.slot_map.tolist() == c["slot_map"]
    assert pl.src_index.tolist() == c["src_index"]
    assert pl.n_overflow == c["n_overflow"]
    assert check_plan(topk, c["R"], c["S"], c["E"], c["K"], c["B"], c["mode"],
                      pl.cu_seqlens, pl.replica_expert, pl.slot_map, pl.src_index) == []


def test_maxvio_hand_values():
    # T = [4,0,0,0] over R*S*K = 4 slots and E = 4: Tbar = 1, maxvio = 4/1 - 1 = 3.
    assert P.maxvio(np.array([4, 0, 0, 0]), 1, 4, 1, 4) == pytest.approx(3.0)
    # perfectly balanced routing
    assert P.maxvio(np.array([2, 2, 2, 2]), 2, 2, 2, 4) == pytest.approx(0.0)
    # Tbar need not be an integer: 3 experts, 12 slots -> Tbar 4; T max 7 -> 0.75
    assert P.maxvio(np.array([5, 7, 0]), 3, 4, 1, 3) == pytest.approx(0.75)
    # bench shape: Tbar = 8*8192*8/384 = 1365.33...; T max 2731 -> 1.000244...
    assert P.maxvio(np.array([2731] + [0] * 383), 8, 8192, 8, 384) == pytest.approx(2731 / (65536 * 8 / 384) - 1)


def _slot_rank_literal(flat):
    """t(u) = #{u' < u : e(u') = e(u)}, written as the double loop of its definition."""
    return [sum(1 for v in range(u) if flat[v] == flat[u]) for u in range(len(flat))]


def _dest_row(pl, R, S, K, E, B, u):
    SK = S * K
    q, pos = divmod(int(pl.slot_map[u]), SK)
    cu = pl.cu_seqlens[q]
    row = max(i for i in range(E + B) if cu[i] <= pos and cu[i] < cu[i + 1])
    return q, row, pos - cu[row]


def test_slot_rank_matches_definition():
    rng = np.random.default_rng(3)
    R, S, E, K, B = 2, 6, 6, 2, 3
    topk = np.stack([rng.choice(E, K, replace=False) for _ in range(R * S)]).astype(np.int32)
    pl = P.plan(topk, R, S, E, K, B, "train")
    flat = topk.reshape(-1).tolist()
    t = _slot_rank_literal(flat)
    # inside a piece, consecutive t land on consecutive positions of one row
    for e in range(E):
        for q, row, t_lo, t_hi in pl.pieces[e]:
            us = [u for u in range(len(flat)) if flat[u] == e and t_lo <= t[u] < t_hi]
            assert [_dest_row(pl, R, S, K, E, B, u)[:2] for u in us] == [(q, row)] * len(us)
            offs = [_dest_row(pl, R, S, K, E, B, u)[2] for u in us]
            assert offs == sorted(offs) and offs[-1] - offs[0] == len(us) - 1


def test_single_rank_is_stable_counting_sort():
    """R = 1: every expert is home, so the plan is the stable counting sort of the
    flat expert ids; rows E..E+B-1 stay empty."""
    rng = np.random.default_rng(0)
    S, E, K = 50, 7, 3
    topk = np.stack([rng.choice(E, K, replace=False) for _ in range(S)]).astype(np.int32)
    pl = P.plan(topk, 1, S, E, K, E, "train")
    flat = topk.reshape(-1)
    assert pl.slot_map.tolist() == np.argsort(np.argsort(flat, kind="stable"), kind="stable").tolist()
    counts = np.bincount(flat, minlength=E)
    assert pl.cu_seqlens[0].tolist() == [0] + np.cumsum(counts).tolist() + [S * K] * E
    assert (pl.replica_expert == -1).all() and pl.parent == [-1]


def test_balanced_routing_needs_no_replicas():
    R, S, E, K = 4, 8, 8, 2
    G = E // R
    # token s of rank r picks both experts of group (r + s) % R: each group gets SK
    topk = np.array([[((r + s) % R) * G, ((r + s) % R) * G + 1] for r in range(R) for s in range(S)],
                    dtype=np.int32)
    pl = P.plan(topk, R, S, E, K, G, "train")
    assert pl.L == [S * K] * R
    assert (pl.replica_expert == -1).all() and pl.n_overflow == 0
    assert pl.parent == [-1] * R


def test_single_hot_group_is_a_star():
    """Everything routed to group 0: rank 0 is the only donor and every other rank
    fills its whole S*K buffer with replicas of group 0's experts."""
    R, S, E, K = 4, 6, 8, 2
    G = E // R
    rng = np.random.default_rng(1)
    topk = np.stack([rng.choice(G, K, replace=False) for _ in range(R * S)]).astype(np.int32)
    pl = P.plan(topk, R, S, E, K, G, "train")
    SK = S * K
    assert pl.parent == [-1] + [0] * (R - 1)
    for q in range(1, R):
        lens = np.diff(pl.cu_seqlens[q])
        assert lens[E:].sum() == SK and lens[:E].sum() == 0
        assert all(0 <= e < G for e in pl.replica_expert[q] if e >= 0)
    assert check_plan(topk, R, S, E, K, G, "train", pl.cu_seqlens, pl.replica_expert,
                      pl.slot_map, pl.src_index) == []


def _all_routings(N, E, K):
    combos = list(itertools.combinations(range(E), K))
    for choice in itertools.product(range(len(combos)), repeat=N):
        yield np.array([combos[c] for c in choice], dtype=np.int32)


EXHAUSTIVE = [(2, 2, 4, 1), (2, 2, 4, 2), (3, 2, 3, 1), (3, 1, 6, 2), (2, 3, 4, 2)]


@pytest.mark.parametrize("R,S,E,K", EXHAUSTIVE)
def test_exhaustive_tiny_routings(R, S, E, K):
    """Every routing of the shape, training mode and every inference B in 0..G."""
    G = E // R
    n = 0
    for topk in _all_routings(R * S, E, K):
        for mode, B in [("train", G)] + [("infer", b) for b in range(G + 1)]:
            pl = P.plan(topk, R, S, E, K, B, mode)
            bad = check_plan(topk, R, S, E, K, B, mode, pl.cu_seqlens, pl.replica_expert,
                             pl.slot_map, pl.src_index)
            assert bad == [], (topk.tolist(), mode, B, bad)
            assert check_order(pl.cu_seqlens, pl.src_index, R, S, K, E, B) == []
            assert pl.n_replicas <= R * B
        n += 1
    assert n == len(list(itertools.combinations(range(E), K))) ** (R * S)


def test_donor_tree_properties_random_loads():
    """Random load vectors up to 64 ranks: one parent per rank, every rank ends at
    exactly SK, receipts <= need <= SK, gifts <= own load."""
    rng = np.random.default_rng(7)
    for _ in range(3000):
        R = int(rng.integers(1, 65))
        SK = int(rng.integers(1, 50))
        # random composition of R*SK into R parts
        cuts = np.sort(rng.integers(0, R * SK + 1, size=R - 1))
        L = np.diff(np.concatenate([[0], cuts, [R * SK]])).tolist()
        parent, gifts = P.donor_tree(L, SK)
        recv = [0] * R
        give = [0] * R
        for p in range(R):
            for c, a in gifts[p]:
                assert parent[c] == p and a > 0
                recv[c] += a
                give[p] += a
        for p in range(R):
            assert L[p] - give[p] + recv[p] == SK
            assert recv[p] <= SK and give[p] <= L[p]
            if L[p] <= SK:
                assert give[p] == 0          # only hot ranks donate
        # a rank receives from exactly its parent, once
        for c in range(R):
            assert sum(1 for p in range(R) for cc, _ in gifts[p] if cc == c) == (parent[c] >= 0)


def _valid_plan_small():
    topk = np.array([[0], [0], [1], [0]], dtype=np.int32)
    pl = P.plan(topk, 2, 2, 4, 1, 2, "train")
    return topk, pl


def test_checker_rejects_planted_mistakes():
    """Plant one mistake at a time in a valid plan: the checker must catch each."""
    topk, pl = _valid_plan_small()
    args = (topk, 2, 2, 4, 1, 2, "train")
    ok = (pl.cu_seqlens, pl.replica_expert, pl.slot_map, pl.src_index)
    assert check_plan(*args, *ok) == []
    # swap the destinations of slots of different experts
    sm = pl.slot_map.copy(); sm[[0, 2]] = sm[[2, 0]]
    si = np.argsort(sm).astype(np.int32)
    assert any(b.startswith("I3") for b in check_plan(*args, pl.cu_seqlens, pl.replica_expert, sm, si))
    # wrong replica id
    rep = pl.replica_expert.copy(); rep[1, 0] = 1
    assert check_plan(*args, pl.cu_seqlens, rep, pl.slot_map, pl.src_index)
    # a rank with one slot too many
    cu = pl.cu_seqlens.copy(); cu[1, -1] += 1
    assert any(b.startswith("I1") for b in check_plan(*args, cu, pl.replica_expert, pl.slot_map, pl.src_index))
    # duplicated destination
    sm = pl.slot_map.copy(); sm[1] = sm[0]
    assert any(b.startswith("I2") for b in check_plan(*args, pl.cu_seqlens, pl.replica_expert, sm, pl.src_index))
    # src_index not the inverse
    si = pl.src_index.copy(); si[[0, 1]] = si[[1, 0]]
    assert any(b.startswith("I2") for b in check_plan(*args, pl.cu_seqlens, pl.replica_expert, pl.slot_map, si))
    # a replica of a home expert
    rep = pl.replica_expert.copy(); rep[0, 0] = 0
    cu = pl.cu_seqlens.copy()
    assert check_plan(*args, cu, rep, pl.slot_map, pl.src_index)


def test_checker_rejects_two_remote_groups_and_training_overflow():
    # R=3, G=1: rank 2 serves one slot from e0 (row 3 slot) and one from e1 (home row 1,
    # an overflow row): two remote groups, and overflow in training.
    R, S, E, K, B = 3, 2, 3, 1, 1
    topk = np.array([[0], [0], [0], [1], [1], [1]], dtype=np.int32)
    # rank 0: e0 x2 ; rank 1: e1 x2 ; rank 2: e0 (slot) + e1 (home row read remotely)
    cu = np.array([[0, 2, 2, 2, 2], [0, 0, 2, 2, 2], [0, 0, 1, 1, 2]], dtype=np.int32)
    rep = np.array([[-1], [-1], [0]], dtype=np.int32)
    # u: 0,1 -> rank 0 rows; 2 -> rank 2 slot (pos 1); 3 -> rank 2 row 1 (pos 0); 4,5 -> rank 1
    sm = np.array([0, 1, 5, 4, 2, 3], dtype=np.int32)
    si = np.argsort(sm).astype(np.int32)
    bad = check_plan(topk, R, S, E, K, B, "train", cu, rep, sm, si)
    assert any(b.startswith("I5") for b in bad)
    assert any(b.startswith("I6") for b in bad)


def test_order_checker_rejects_unstable_segment():
    topk = np.array([[0], [0], [1], [0]], dtype=np.int32)
    pl = P.plan(topk, 2, 2, 4, 1, 2, "train")
    # rank 1's slot row holds u=0,1 in that order; swap them
    sm = pl.slot_map.copy(); sm[[0, 1]] = sm[[1, 0]]
    si = np.argsort(sm).astype(np.int32)
    assert check_plan(topk, 2, 2, 4, 1, 2, "train", pl.cu_seqlens, pl.replica_expert, sm, si) == []
    assert check_order(pl.cu_seqlens, si, 2, 2, 1, 4, 2) != []


# ----------------------------------------------------------------- plain-EP loads

@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_home_only_loads_hand_worked(case):
    """Rows each rank computes with no redundant experts (plain EP: every slot goes
    to its expert's home rank), against the loads worked by hand in each case."""
    c = case
    topk = np.array(c["topk_idx"], dtype=np.int32)
    assert P.home_only_loads(topk, c["R"], c["E"]) == c["L"]


def test_home_only_loads_brute_force():
    """Against a literal count: visit every (token, k) slot and credit the rank that
    owns its expert (e // (E/R)); the loads add up to every slot, and the balanced
    plan starts from the same loads and ends with exactly S*K on every rank."""
    rng = np.random.default_rng(11)
    for _ in range(40):
        R = int(rng.integers(1, 7))
        G = int(rng.integers(1, 5))
        E = R * G
        K = int(rng.integers(1, min(E, 4) + 1))
        S = int(rng.integers(0, 9))
        p = rng.dirichlet(np.full(E, 0.3))
        topk = np.array([rng.choice(E, K, replace=False, p=p) for _ in range(R * S)],
                        dtype=np.int32).reshape(R * S, K)
        want = [0] * R
        for g in range(R * S):
            for k in range(K):
                want[int(topk[g, k]) // G] += 1
        got = P.home_only_loads(topk, R, E)
        assert got == want
        assert sum(got) == R * S * K
        pl = P.plan(topk, R, S, E, K, G, "train")
        assert list(pl.L) == want
        assert all(int(pl.cu_seqlens[q, -1]) == S * K for q in range(R))
