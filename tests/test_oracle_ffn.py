"""Pins of the expert-FFN oracle (oracle/ffn.py) against hand values, closed
forms, finite differences and torch's own silu and autograd.

* the interleaved gate/up column layout against literal index lists;
* silu at points with exact sigmoids (sigmoid(ln 3) = 3/4) and its limits;
* silu' against central differences of silu;
* swiglu and its backward against torch.nn.functional.silu and autograd;
* the dense FFN forward against a closed form (one-hot tokens select one row of
  W1, constant gate and up values, W2 with a known product);
* the dense FFN backward against torch autograd (float64) of the same loss;
* the plan-based FFN pipeline against the dense result for every prefetch
  budget B, and the two weight gradients (home plus replicas after reduce_grad)
  against the dense ones;
* the column-selective sampled helpers against the full dense gradients.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ffn as FF
from oracle import moe as M
from oracle import plan as P


def test_gate_up_columns_literal():
    g, u = FF.gate_up_columns(64)
    assert g.tolist() == list(range(0, 32)) + list(range(64, 96))
    assert u.tolist() == list(range(32, 64)) + list(range(96, 128))
    g, u = FF.gate_up_columns(32)
    assert g.tolist() == list(range(32)) and u.tolist() == list(range(32, 64))
    # a permutation of all 2H' columns
    g, u = FF.gate_up_columns(1408)
    assert sorted(g.tolist() + u.tolist()) == list(range(2816))


def test_silu_exact_points_and_limits():
    l3 = math.log(3.0)
    assert FF.silu(0.0) == 0.0
    assert abs(FF.silu(l3) - 0.75 * l3) < 1e-15
    assert abs(FF.silu(-l3) + 0.25 * l3) < 1e-15
    assert abs(FF.silu(40.0) - 40.0) < 1e-12
    assert abs(FF.silu(-40.0)) < 1e-15
    assert abs(FF.silu_grad(0.0) - 0.5) < 1e-15
    # sigmoid(ln 3) = 3/4: silu'(ln 3) = 3/4 (1 + ln3 / 4)
    assert abs(FF.silu_grad(l3) - 0.75 * (1.0 + l3 / 4.0)) < 1e-15
    assert abs(FF.silu(-800.0)) == 0.0


def test_silu_grad_matches_central_differences():
    v = np.linspace(-12.0, 12.0, 481)
    eps = 1e-6
    fd = (FF.silu(v + eps) - FF.silu(v - eps)) / (2 * eps)
    assert np.abs(FF.silu_grad(v) - fd).max() < 1e-8


def test_swiglu_and_backward_match_torch():
    rng = np.random.default_rng(0)
    Hp = 96
    h = rng.standard_normal((7, 2 * Hp)) * 3.0
    da = rng.standard_normal((7, Hp))
    gate, up = FF.gate_up_columns(Hp)
    ht = torch.tensor(h, requires_grad=True)
    act_t = F.silu(ht[:, torch.from_numpy(gate)]) * ht[:, torch.from_numpy(up)]
    (act_t * torch.tensor(da)).sum().backward()
    assert np.allclose(FF.swiglu(h, None), act_t.detach().numpy(), rtol=1e-14, atol=1e-14)
    assert np.allclose(FF.swiglu_backward(h, da, None), ht.grad.numpy(), rtol=1e-13, atol=1e-13)


def test_roundings_are_bf16_of_float32():
    h = np.array([[1.0 + 2.0 ** -9, 3.0, -0.7, 1e-3] * 16 + [0.25] * 64], dtype=np.float64)
    act = FF.swiglu(h, "bf16")
    ref = torch.tensor(FF.swiglu(h, None)).float().to(torch.bfloat16).double().numpy()
    assert np.array_equal(act, ref)
    assert np.array_equal(FF.round_to(h, "fp32"), h.astype(np.float32).astype(np.float64))


def _layer(R, S, E, K, H, Hp, seed, hot_group=0, weight=8.0):
    rng = np.random.default_rng(seed)
    G = E // R
    p = np.ones(E)
    p[hot_group * G:(hot_group + 1) * G] = weight
    p /= p.sum()
    topk = np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(R * S)]).astype(np.int32)
    gates = rng.random((R * S, K)).astype(np.float32)
    x = M.bf16_round(rng.standard_normal((R * S, H)).astype(np.float32))
    W1 = M.bf16_round((rng.standard_normal((E, H, 2 * Hp)) / math.sqrt(H)).astype(np.float32))
    W2 = M.bf16_round((rng.standard_normal((E, Hp, H)) / math.sqrt(Hp)).astype(np.float32))
    return rng, topk, gates, x, W1, W2


def test_dense_ffn_forward_closed_form():
    """One-hot token rows x[g] = c_g * e_{r(g)} make h a scaled row of W1[e]. With
    that row's gate entries ln 3 and up entries 2, act = c silu(c ln3) * 2 per
    column, and W2[e][p, j] = (p + 1) (j + 1) gives z_j = act (j+1) sum(p+1)."""
    E, K, H, Hp, N = 3, 2, 5, 64, 6
    rng = np.random.default_rng(2)
    topk = np.stack([rng.choice(E, K, replace=False) for _ in range(N)]).astype(np.int32)
    gates = rng.random((N, K)).astype(np.float32)
    rows = rng.integers(0, H, N)
    c = rng.choice([0.5, 1.0, 2.0], N)
    x = np.zeros((N, H))
    x[np.arange(N), rows] = c
    gate, up = FF.gate_up_columns(Hp)
    W1 = rng.standard_normal((E, H, 2 * Hp))
    for e in range(E):
        for r in range(H):
            W1[e, r, gate] = math.log(3.0) * (e + 1)
            W1[e, r, up] = 2.0
    W2 = np.einsum("p,j->pj", np.arange(1, Hp + 1.0), np.arange(1, H + 1.0))
    W2 = np.broadcast_to(W2, (E, Hp, H))
    y = FF.dense_ffn_forward(x, W1, W2, topk, gates, None)
    sum_p = Hp * (Hp + 1) / 2
    for g in range(N):
        want = np.zeros(H)
        for k in range(K):
            e = topk[g, k]
            v = c[g] * math.log(3.0) * (e + 1)
            act = v / (1 + math.exp(-v)) * 2.0 * c[g]
            want += gates[g, k] * act * sum_p * np.arange(1, H + 1.0)
        assert np.allclose(y[g], want, rtol=1e-13)


def test_dense_ffn_backward_matches_autograd():
    R, S, E, K, H, Hp = 2, 6, 4, 2, 7, 64
    rng, topk, gates, x, W1, W2 = _layer(R, S, E, K, H, Hp, seed=3)
    dy = rng.standard_normal((R * S, H)).astype(np.float32)
    d = M.gated_dy(dy, gates, "fp32")
    dx, dW1, dW2 = FF.dense_ffn_backward(x, W1, W2, topk, d, None)
    gate, up = FF.gate_up_columns(Hp)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    W1t = torch.tensor(W1, dtype=torch.float64, requires_grad=True)
    W2t = torch.tensor(W2, dtype=torch.float64, requires_grad=True)
    dt = torch.tensor(d, dtype=torch.float64)
    loss = 0
    for g in range(R * S):
        for k in range(K):
            e = int(topk[g, k])
            h = xt[g] @ W1t[e]
            z = (F.silu(h[torch.from_numpy(gate)]) * h[torch.from_numpy(up)]) @ W2t[e]
            loss = loss + (z * dt[g * K + k]).sum()
    loss.backward()
    assert np.allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert np.allclose(dW1, W1t.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert np.allclose(dW2, W2t.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("mode_B", [("train", None), ("infer", 0), ("infer", 1)])
@pytest.mark.parametrize("dtype", [None, "bf16"])
def test_ffn_pipeline_equals_dense_for_every_B(mode_B, dtype):
    mode, B = mode_B
    R, S, E, K, H, Hp = 4, 12, 12, 3, 8, 32
    G = E // R
    B = G if B is None else B
    rng, topk, gates, x, W1, W2 = _layer(R, S, E, K, H, Hp, seed=5)
    pl = P.plan(topk, R, S, E, K, B, mode)
    assert pl.n_replicas + pl.n_overflow > 0
    y, act = FF.pipeline_ffn_forward(x, W1, W2, topk, gates, pl, R, S, E, K, B, dtype)
    ref = FF.dense_ffn_forward(x, W1, W2, topk, gates, dtype)
    # float64 pipelines agree to rounding order; with bfloat16 roundings a product
    # landing within rounding-order distance of a tie may round the other way
    tol = 1e-12 if dtype is None else 1e-3
    assert np.abs(y - ref).max() <= tol * np.abs(ref).max()
    # buffer row i holds the slot src_index[i] names
    for i in (0, S * K - 1, R * S * K - 1):
        u = int(np.asarray(pl.src_index).ravel()[i])
        e = topk[u // K, u % K]
        want = FF.swiglu(x[u // K][None].astype(np.float64) @ W1[e], dtype)[0]
        assert np.allclose(act[i], want, rtol=1e-12, atol=1e-12 if dtype is None else 0.02)


def test_ffn_pipeline_backward_gradients_fold_home():
    R, S, E, K, H, Hp = 4, 12, 8, 2, 8, 32
    G = E // R
    rng, topk, gates, x, W1, W2 = _layer(R, S, E, K, H, Hp, seed=9, hot_group=1, weight=10.0)
    dy = M.bf16_round(rng.standard_normal((R * S, H)).astype(np.float32))
    pl = P.plan(topk, R, S, E, K, G, "train")
    assert pl.n_replicas > 0
    SK = S * K
    dtype = None
    d = M.gated_dy(dy, gates, "bf16")
    dx_ref, dW1_ref, dW2_ref = FF.dense_ffn_backward(x, W1, W2, topk, d, dtype)

    W1a = M.prefetch(W1, pl.replica_expert, E, G)
    W2a = M.prefetch(W2, pl.replica_expert, E, G)
    xp = M.permute(x, pl.slot_map, K)
    h = M.segment_matmul(xp, W1a, pl.cu_seqlens, R, SK, E, G)
    act = FF.swiglu(h, dtype)
    dyp = M.permute(d, pl.slot_map, K, per_slot=True)
    da = M.segment_matmul(dyp, W2a, pl.cu_seqlens, R, SK, E, G, transpose_w=True)
    g2 = np.zeros((E, Hp, H)); r2 = np.zeros((R, G, Hp, H))
    M.segment_wgrad(act, dyp, pl.cu_seqlens, R, SK, E, G, g2, r2)
    dh = FF.swiglu_backward(FF.round_to(h, dtype), da, dtype)
    dxp = M.segment_matmul(dh, W1a, pl.cu_seqlens, R, SK, E, G, transpose_w=True)
    g1 = np.zeros((E, H, 2 * Hp)); r1 = np.zeros((R, G, H, 2 * Hp))
    M.segment_wgrad(xp, dh, pl.cu_seqlens, R, SK, E, G, g1, r1)
    dx = M.combine(dxp, pl.slot_map, None, R * S, K)
    assert np.abs(r1).sum() > 0 and np.abs(r2).sum() > 0
    M.reduce_grad(pl.replica_expert, r1, g1)
    M.reduce_grad(pl.replica_expert, r2, g2)
    assert not r1.any() and not r2.any()
    assert np.abs(dx - dx_ref).max() <= 1e-12 * np.abs(dx_ref).max()
    assert np.abs(g1 - dW1_ref).max() <= 1e-12 * np.abs(dW1_ref).max()
    assert np.abs(g2 - dW2_ref).max() <= 1e-12 * np.abs(dW2_ref).max()


@pytest.mark.parametrize("dtype", [None, "bf16"])
def test_sampled_helpers_match_dense(dtype):
    R, S, E, K, H, Hp = 2, 8, 4, 2, 9, 64
    rng, topk, gates, x, W1, W2 = _layer(R, S, E, K, H, Hp, seed=11)
    dy = M.bf16_round(rng.standard_normal((R * S, H)).astype(np.float32))
    d = M.gated_dy(dy, gates, "bf16")
    dx_ref, dW1_ref, dW2_ref = FF.dense_ffn_backward(x, W1, W2, topk, d, dtype)
    y_ref = FF.dense_ffn_forward(x, W1, W2, topk, gates, dtype)
    g = 3
    y = sum(float(gates[g, k]) * FF.slot_values(x[g], W1[topk[g, k]], W2[topk[g, k]], dtype)[2]
            for k in range(K))
    assert np.allclose(y, y_ref[g], rtol=1e-12, atol=1e-12)
    dx = sum(FF.slot_backward(x[g], d[g * K + k], W1[topk[g, k]], W2[topk[g, k]], dtype)[1]
             for k in range(K))
    assert np.allclose(dx, dx_ref[g], rtol=1e-12, atol=1e-12)
    e = 1
    tok, kk = np.nonzero(topk == e)
    hh, pp = np.array([0, 4, 8]), np.array([1, 33, 63])
    dW1, dW2 = FF.wgrad_entries_ffn(x[tok], d[tok * K + kk], W1[e], W2[e], hh, pp, dtype)
    gate, up = FF.gate_up_columns(Hp)
    assert np.allclose(dW1[:, 0], dW1_ref[e][np.ix_(hh, gate[pp])], rtol=1e-12, atol=1e-12)
    assert np.allclose(dW1[:, 1], dW1_ref[e][np.ix_(hh, up[pp])], rtol=1e-12, atol=1e-12)
    assert np.allclose(dW2, dW2_ref[e][pp], rtol=1e-12, atol=1e-12)
