"""Plan invariants.  TEST INFRASTRUCTURE (see oracle/__init__.py).

``check_plan`` knows nothing of the planner rule in ``oracle.plan``: it accepts
any plan that has the properties the pages state, and returns the list of
violated properties (empty = valid).

  I1  every rank receives exactly S*K slots: cu[q][0] = 0, cu nondecreasing,
      cu[q][E+B] = S*K  [maestro "The core idea: dynamic redundant experts"]
  I2  slot_map is a bijection of the R*S*K slots onto the R*(S*K) buffer rows and
      src_index is its inverse (each (token, k) served exactly once)
  I3  a slot that lands in row i of rank q is served by its own expert: i < E
      means i is that expert; i >= E means replica_expert[q][i-E] is that expert
      [maestro "The memory contract": rows [0,E) home experts, [E,E+B) slots]
  I4  a used prefetch slot holds a remote expert and has rows; an unused slot
      (-1) has none; no expert twice on one rank
  I5  remote experts of one rank (slots or overflow rows) all come from one
      home group [maestro "The memory contract"]
  I6  training: B = E/R and no overflow rows, so every touched expert is local;
      inference: overflow rows only once all B slots are used
  I7  within a row segment, slots keep ascending flat slot id (the stated order
      of the zero-copy buffer; the pages fix no order, so this is a chosen
      reading, checked separately by ``check_order``)
"""
from __future__ import annotations

import numpy as np


def check_plan(topk_idx, R, S, E, K, B, mode, cu_seqlens, replica_expert,
               slot_map, src_index) -> list[str]:
    bad: list[str] = []
    G = E // R
    SK = S * K
    n = R * S * K
    flat = np.asarray(topk_idx).reshape(-1).astype(np.int64)
    cu = np.asarray(cu_seqlens).astype(np.int64)
    rep = np.asarray(replica_expert).astype(np.int64)
    sm = np.asarray(slot_map).astype(np.int64)
    si = np.asarray(src_index).astype(np.int64)

    if cu.shape != (R, E + B + 1) or rep.shape != (R, B) or sm.shape != (n,) or si.shape != (n,):
        return ["shapes"]
    # I1
    for q in range(R):
        if cu[q, 0] != 0 or cu[q, E + B] != SK:
            bad.append(f"I1 rank {q} total {cu[q, E + B] - cu[q, 0]} != {SK}")
        if (np.diff(cu[q]) < 0).any():
            bad.append(f"I1 rank {q} cu_seqlens decreasing")
    # I2
    if n and (sm.min() < 0 or sm.max() >= n or len(set(sm.tolist())) != n):
        bad.append("I2 slot_map not a bijection")
        return bad
    for u in range(n):
        if si[sm[u]] != u:
            bad.append(f"I2 src_index[slot_map[{u}]] != {u}")
            break
    # row of each destination
    row_of = np.empty(n, dtype=np.int64)
    for q in range(R):
        for i in range(E + B):
            row_of[q * SK + cu[q, i]: q * SK + cu[q, i + 1]] = i
    # I3
    for u in range(n):
        q, i = divmod(int(sm[u]), SK)[0], int(row_of[sm[u]])
        e = int(flat[u])
        served = i if i < E else int(rep[q, i - E])
        if served != e:
            bad.append(f"I3 slot {u} (expert {e}) served by {served} on rank {q} row {i}")
            break
    # I4, I5, I6
    for q in range(R):
        lens = np.diff(cu[q])
        used = [j for j in range(B) if rep[q, j] >= 0]
        for j in range(B):
            if rep[q, j] >= 0 and lens[E + j] == 0:
                bad.append(f"I4 rank {q} slot {j} holds {rep[q, j]} but has no rows")
            if rep[q, j] < 0 and lens[E + j] != 0:
                bad.append(f"I4 rank {q} unused slot {j} has rows")
            if rep[q, j] >= 0 and rep[q, j] // G == q:
                bad.append(f"I4 rank {q} slot {j} duplicates a home expert")
        if len(set(int(rep[q, j]) for j in used)) != len(used):
            bad.append(f"I4 rank {q} holds an expert twice")
        overflow = [i for i in range(E) if lens[i] > 0 and i // G != q]
        if set(overflow) & set(int(rep[q, j]) for j in used):
            bad.append(f"I4 rank {q} reads an expert both from a slot and its home row")
        groups = {int(rep[q, j]) // G for j in used} | {i // G for i in overflow}
        if len(groups) > 1:
            bad.append(f"I5 rank {q} draws from groups {sorted(groups)}")
        if mode == "train" and overflow:
            bad.append(f"I6 rank {q} reads remote rows {overflow} in training")
        if mode == "infer" and overflow and len(used) < B:
            bad.append(f"I6 rank {q} overflows with free slots")
    if mode == "train" and B != G:
        bad.append("I6 training needs B = E/R")
    return bad


def check_order(cu_seqlens, src_index, R, S, K, E, B) -> list[str]:
    """I7: ascending flat slot id inside every row segment."""
    bad = []
    SK = S * K
    cu = np.asarray(cu_seqlens).astype(np.int64)
    si = np.asarray(src_index).astype(np.int64)
    for q in range(R):
        for i in range(E + B):
            seg = si[q * SK + cu[q, i]: q * SK + cu[q, i + 1]]
            if (np.diff(seg) <= 0).any():
                bad.append(f"I7 rank {q} row {i} not ascending")
    return bad
