"""Property-based pins of the oracle on randomised small layers (hypothesis).

Hypothesis draws a shape (ranks, experts per rank, K, tokens per rank, mode and
B) and a routing (K distinct experts per token, from a skewed distribution so
replicas and overflow occur), and checks:

* the plan against the invariant checker, which does not know the planner rule:
  exactly S*K slots per rank, a bijection between slots and (token, k), every slot
  served by its expert's home row or a replica of it, replicas from at most one
  remote home group in training, the B rules [ai-maestro.online "Moonshot AI
  open-sources MoonEP", sections "The core idea" and "The memory contract"];
* the stable order of every segment (global token order);
* the float64 pipeline (prefetch, permute, segment products, gated combine) against
  the plan-free dense definition y[g] = sum_k gate[g,k] x[g] W[topk[g,k]], and so
  its independence of B (the B setting does not change the results: same page,
  "The memory contract");
* in training, the backward pipeline (gated dY, segment dgrad and wgrad, unpermute,
  reduce_grad) against the dense gradients, with the consumed slots left at zero.

The draws are derandomized (a fixed seed per test), so every run checks the same
examples; ten times as many draws also passed when these tests were written.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import moe as M
from oracle import plan as P
from oracle.check import check_order, check_plan


@st.composite
def layers(draw):
    R = draw(st.integers(1, 6))
    G = draw(st.integers(1, 5))
    E = R * G
    K = draw(st.integers(1, min(E, 4)))
    S = draw(st.integers(0, 12))
    train = draw(st.booleans())
    B = G if train else draw(st.integers(0, G))
    seed = draw(st.integers(0, 2**31 - 1))
    hot = draw(st.floats(1.0, 30.0))
    return R, S, E, K, B, "train" if train else "infer", seed, hot


def _routing(R, S, E, K, seed, hot):
    rng = np.random.default_rng(seed)
    p = np.ones(E)
    p[rng.integers(0, E)] = hot          # one hot expert drives skew
    p /= p.sum()
    rows = [rng.choice(E, K, replace=False, p=p) for _ in range(R * S)]
    topk = np.array(rows, dtype=np.int32).reshape(R * S, K)
    gates = rng.random((R * S, K)).astype(np.float32)
    return topk, gates, rng


@settings(max_examples=300, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(layers())
def test_plan_invariants_and_order(layer):
    R, S, E, K, B, mode, seed, hot = layer
    topk, _, _ = _routing(R, S, E, K, seed, hot)
    pl = P.plan(topk, R, S, E, K, B, mode)
    bad = check_plan(topk, R, S, E, K, B, mode, pl.cu_seqlens, pl.replica_expert, pl.slot_map,
                     pl.src_index)
    assert bad == [], bad
    assert check_order(pl.cu_seqlens, pl.src_index, R, S, K, E, B) == []
    assert pl.n_replicas <= R * B


@settings(max_examples=120, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(layers(), st.integers(1, 9), st.integers(1, 9))
def test_pipeline_equals_dense_definition(layer, H, Hp):
    R, S, E, K, B, mode, seed, hot = layer
    topk, gates, rng = _routing(R, S, E, K, seed, hot)
    x = rng.standard_normal((R * S, H))
    W = rng.standard_normal((E, H, Hp))
    pl = P.plan(topk, R, S, E, K, B, mode)
    SK = S * K
    W_all = M.prefetch(W, pl.replica_expert, E, B)
    xp = M.permute(x, pl.slot_map, K)
    out = M.segment_matmul(xp, W_all, pl.cu_seqlens, R, SK, E, B)
    y = M.combine(out, pl.slot_map, gates, R * S, K)
    ref = M.dense_forward(x, W, topk, gates)
    assert np.abs(y - ref).max(initial=0.0) <= 1e-12 * max(np.abs(ref).max(initial=0.0), 1.0)
    if mode != "train" or S == 0:
        return
    dy = rng.standard_normal((R * S, Hp))
    d = M.gated_dy(dy, gates, None)
    dx_ref, dW_ref = M.dense_backward(x, W, topk, d)
    dyp = M.permute(d, pl.slot_map, K, per_slot=True)
    dxp = M.segment_matmul(dyp, W_all, pl.cu_seqlens, R, SK, E, B, transpose_w=True)
    dx = M.combine(dxp, pl.slot_map, None, R * S, K)
    grad_home = np.zeros((E, H, Hp))
    reduce_buf = np.zeros((R, B, H, Hp))
    M.segment_wgrad(xp, dyp, pl.cu_seqlens, R, SK, E, B, grad_home, reduce_buf)
    M.reduce_grad(pl.replica_expert, reduce_buf, grad_home)
    assert not np.any(reduce_buf)
    scale = max(np.abs(dW_ref).max(initial=0.0), 1.0)
    assert np.abs(dx - dx_ref).max(initial=0.0) <= 1e-12 * max(np.abs(dx_ref).max(initial=0.0), 1.0)
    assert np.abs(grad_home - dW_ref).max(initial=0.0) <= 1e-12 * scale
