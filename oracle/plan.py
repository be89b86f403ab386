"""Oracle of the redundant-expert plan.  TEST INFRASTRUCTURE (see oracle/__init__.py).

What the pages fix:
  * every rank receives exactly S*K token-slots whatever the skew, obtained by
    serving some slots from duplicated ("redundant") experts planned from the
    current router output [maestro "The core idea: dynamic redundant experts";
    noticiai "A ideia central"];
  * the expert-compute view is one [E+B, H, H'] tensor: rows [0,E) are the home
    experts, E/R per rank, rows [E,E+B) are the rank's prefetch slots; a per-rank
    cu_seqlens over those E+B rows selects the active rows [maestro "The memory
    contract"; spaxe para. 6-7];
  * training uses B = E/R and duplicates experts of at most one remote home group
    per rank; inference may use B < E/R, and experts beyond the B slots are read
    from their home rows [maestro "The memory contract"; spaxe para. 7-8];
  * tokens go straight to their expert-grouped positions of a fixed S*K buffer
    [maestro "The core idea"].

What the pages leave open, and the reading taken here (the planner is called
"near-optimal" but never specified):
  P1  T_e = #slots routed to e; L_p = sum of T_e over rank p's home experts.
  P2  Donor tree: hot ranks (L_p > SK) and cold ranks (L_p < SK), both in
      ascending id.  A cursor walks the hot list; each cold rank takes all it
      needs from the current hot rank; when that rank's surplus goes negative it
      becomes a child of the next hot rank, which covers the deficit.
  P3  A donor orders its home experts by (T_e descending, e ascending) and lays
      their slots end to end.
  P4  Its gifts, in the order they were made, take consecutive ranges of that
      layout from the start; the donor keeps the tail.
  P5  Intersecting each expert's interval with those ranges gives its pieces.
  P6  A child numbers the distinct experts of its range j = 0, 1, ... in layout
      order; j < B gets prefetch row E+j, j >= B reads home row e (overflow).
  P7  Slots of one expert are ranked by flat slot id u = g*K + k (g = global
      token id r*S + s); cu_seqlens is the exclusive prefix of row lengths;
      a slot lands at cu[q][row] + (t - t_lo) of rank q's S*K buffer.
"""
from __future__ import annotations

import dataclasses
import numpy as np


def expert_loads(topk_idx: np.ndarray, E: int) -> np.ndarray:
    """P1: T_e, the number of (token, k) slots routed to expert e.

    [maestro "The problem MoonEP targets"] names T_e the tokens routed to e.
    """
    return np.bincount(np.asarray(topk_idx, dtype=np.int64).reshape(-1), minlength=E)


def maxvio(T: np.ndarray, R: int, S: int, K: int, E: int) -> float:
    """max_e(T_e / Tbar) - 1, Tbar = R*S*K/E, the count every expert would get
    under perfect balance [maestro "The problem MoonEP targets"; noticiai "O
    problema que o MoonEP resolve"].  0 means perfectly balanced."""
    tbar = R * S * K / E
    return max(int(t) for t in T) / tbar - 1.0


def rank_loads(T: np.ndarray, R: int) -> list[int]:
    """P1: L_p = sum of T_e over rank p's home experts e in [p*G, (p+1)*G)."""
    G = len(T) // R
    return [int(sum(int(T[e]) for e in range(p * G, (p + 1) * G))) for p in range(R)]


def donor_tree(L: list[int], SK: int):
    """P2: parent of each rank (-1 = none) and each donor's ordered gift list.

    gifts[p] is a list of (child, amount).  Every rank ends with exactly SK slots:
    cold ranks are filled from the current hot rank; a hot rank whose surplus is
    over-spent takes the deficit from the next hot rank (so it has one parent).
    """
    R = len(L)
    parent = [-1] * R
    gifts: list[list[tuple[int, int]]] = [[] for _ in range(R)]
    hot = [p for p in range(R) if L[p] > SK]
    cold = [q for q in range(R) if L[q] < SK]
    if not hot:
        assert not cold, "loads must sum to R*SK"
        return parent, gifts
    i = 0
    avail = L[hot[0]] - SK
    for q in cold:
        need = SK - L[q]
        parent[q] = hot[i]
        gifts[hot[i]].append((q, need))
        avail -= need
        while avail < 0:
            nxt = hot[i + 1]
            parent[hot[i]] = nxt
            gifts[nxt].append((hot[i], -avail))
            avail += L[nxt] - SK
            i += 1
        if avail == 0 and i + 1 < len(hot):
            i += 1
            avail = L[hot[i]] - SK
    return parent, gifts


@dataclasses.dataclass
class Plan:
    cu_seqlens: np.ndarray       # int32 [R, E+B+1]
    replica_expert: np.ndarray   # int32 [R, B], -1 = unused slot
    slot_map: np.ndarray         # int32 [R*S*K]: u -> q*SK + pos
    src_index: np.ndarray        # int32 [R*S*K]: q*SK + pos -> u
    T: np.ndarray                # int64 [E]
    L: list                      # [R]
    parent: list                 # [R]
    gifts: list                  # [R] lists of (child, amount)
    pieces: list                 # [E] lists of (q, row, t_lo, t_hi), t_lo ascending
    n_replicas: int
    n_overflow: int


def plan(topk_idx: np.ndarray, R: int, S: int, E: int, K: int, B: int, mode: str) -> Plan:
    """The full plan P1-P7 for router output ``topk_idx`` [R*S, K] (int)."""
    G = E // R
    SK = S * K
    assert E % R == 0 and 0 <= B <= G
    assert mode in ("train", "infer")
    if mode == "train":
        assert B == G, "training uses B = E/R [maestro 'The memory contract']"
    flat = [int(v) for v in np.asarray(topk_idx).reshape(-1)]
    assert len(flat) == R * S * K
    assert all(0 <= e < E for e in flat)

    T = expert_loads(flat, E)
    L = rank_loads(T, R)
    parent, gifts = donor_tree(L, SK)

    replica = np.full((R, B), -1, dtype=np.int64)
    counts = np.zeros((R, E + B), dtype=np.int64)
    pieces: list[list[tuple[int, int, int, int]]] = [[] for _ in range(E)]
    n_overflow = 0
    for p in range(R):
        home = list(range(p * G, (p + 1) * G))
        seq = sorted(home, key=lambda e: (-int(T[e]), e))          # P3
        off = {}
        acc = 0
        for e in seq:
            off[e] = acc
            acc += int(T[e])
        ranges = []                                               # P4
        start = 0
        for child, amount in gifts[p]:
            ranges.append((child, start, start + amount))
            start += amount
        ranges.append((p, start, L[p]))                            # home keeps the tail
        for dest, lo, hi in ranges:                                # P5, P6
            j = 0
            for e in seq:
                a = max(lo, off[e])
                b = min(hi, off[e] + int(T[e]))
                if a >= b:
                    continue
                if dest == p:
                    row = e
                else:
                    if j < B:
                        row = E + j
                        replica[dest, j] = e
                    else:
                        row = e            # overflow: home row read in place
                        n_overflow += 1
                    j += 1
                pieces[e].append((dest, row, a - off[e], b - off[e]))
                counts[dest, row] += b - a

    cu = np.zeros((R, E + B + 1), dtype=np.int64)                  # P7
    for q in range(R):
        for row in range(E + B):
            cu[q, row + 1] = cu[q, row] + counts[q, row]
        assert cu[q, E + B] == SK

    seen = [0] * E                      # t = number of earlier slots of the same expert
    slot_map = np.full(R * S * K, -1, dtype=np.int64)
    src_index = np.full(R * S * K, -1, dtype=np.int64)
    for u, e in enumerate(flat):
        t = seen[e]
        seen[e] += 1
        for q, row, t_lo, t_hi in pieces[e]:
            if t_lo <= t < t_hi:
                dest = q * SK + int(cu[q, row]) + (t - t_lo)
                slot_map[u] = dest
                src_index[dest] = u
                break
    assert (slot_map >= 0).all() and (src_index >= 0).all()
    return Plan(cu.astype(np.int32), replica.astype(np.int32), slot_map.astype(np.int32),
                src_index.astype(np.int32), T, L, parent, gifts, pieces,
                int((replica >= 0).sum()), n_overflow)


def home_only_loads(topk_idx: np.ndarray, R: int, E: int) -> list[int]:
    """Rows each rank computes with no redundant experts (plain EP): every slot goes to
    the home rank of its expert, so rank p holds L_p, whatever the skew [maestro "The
    problem MoonEP targets": the hottest rank sets the layer's time]."""
    return rank_loads(expert_loads(topk_idx, E), R)
