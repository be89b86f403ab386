"""Full expert FFN around the plan: gate/up projection, SwiGLU, down projection.
TEST INFRASTRUCTURE.

The pages state the weight contract per projection, an [E+B, H, H'] tensor per
expert weight, with H' the intermediate size of the expert FFN [maestro "The
memory contract"]; they do not name the activation. This oracle takes the usual
gated form of an MoE expert:

  h     = x @ W1[e]                       W1 [E, H, 2H']: gate and up projection
  act   = silu(h_gate) * h_up             silu(v) = v * sigmoid(v) = v / (1 + e^-v)
  z     = act @ W2[e]                     W2 [E, H', H]: down projection
  y[g]  = sum_k gate[g,k] * z(g*K + k)

Gate and up columns of W1 (and of h, and of its gradient) are interleaved in
blocks of BLOCK = 32 columns: intermediate column p has its gate column at
64*(p // 32) + p % 32 and its up column 32 further. The layout is a choice of
this library (so that one 64-column slice of h holds both halves of 32
intermediate columns); any checkpoint is permuted once to it.

Rounding points (the ones the layer performs; everything else is float64):
  act   rounded once to the layer dtype (the down projection's operand);
  hs    h rounded to the layer dtype, saved for the backward pass;
  dh    the SwiGLU gradient, computed from hs and the float32 da, rounded once
        to the layer dtype (the operand of both backward GEMMs of W1).
``dtype=None`` switches every rounding off (pure float64), for the pins.

Backward, with d(u) the gated upstream rows of moe.gated_dy:
  da    = d(u) @ W2[e]^T                          [H']
  dW2[e] += outer(act(u), d(u))
  dh_gate = da * h_up * silu'(h_gate),  dh_up = da * silu(h_gate)
            silu'(v) = s (1 + v (1 - s)),  s = sigmoid(v)
  dx[g] += dh(u) @ W1[e]^T,   dW1[e] += outer(x[g], dh(u))
"""
from __future__ import annotations

import numpy as np

from .moe import bf16_round, combine, permute, prefetch, segment_matmul

BLOCK = 32


def gate_up_columns(Hp: int):
    """(gate, up) column indices of the interleaved [.., 2H'] layout, each [H']."""
    p = np.arange(Hp)
    gate = 2 * BLOCK * (p // BLOCK) + p % BLOCK
    return gate, gate + BLOCK


def round_to(a, dtype):
    """float64 values rounded as the layer stores them: via float32 to bfloat16
    ('bf16'), to float32 ('fp32'), or not at all (None)."""
    a = np.asarray(a, dtype=np.float64)
    if dtype is None:
        return a
    f = a.astype(np.float32)
    return (bf16_round(f) if dtype == "bf16" else f).astype(np.float64)


def sigmoid(v):
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def silu(v):
    v = np.asarray(v, dtype=np.float64)
    return v * sigmoid(v)


def silu_grad(v):
    v = np.asarray(v, dtype=np.float64)
    s = sigmoid(v)
    return s * (1.0 + v * (1.0 - s))


def swiglu(h, dtype):
    """act [n, H'] from h [n, 2H'] (interleaved gate/up columns)."""
    h = np.asarray(h, dtype=np.float64)
    gate, up = gate_up_columns(h.shape[1] // 2)
    return round_to(silu(h[:, gate]) * h[:, up], dtype)


def swiglu_backward(hs, da, dtype):
    """dh [n, 2H'] (interleaved) from the saved pre-activation hs [n, 2H'] and da [n, H']."""
    hs = np.asarray(hs, dtype=np.float64)
    da = np.asarray(da, dtype=np.float64)
    gate, up = gate_up_columns(hs.shape[1] // 2)
    g, u = hs[:, gate], hs[:, up]
    dh = np.zeros_like(hs)
    dh[:, gate] = da * u * silu_grad(g)
    dh[:, up] = da * silu(g)
    return round_to(dh, dtype)


# ----------------------------------------------------------------- dense form

def _slots_of(topk, e):
    tok, kk = np.nonzero(np.asarray(topk) == e)
    return tok, kk


def dense_ffn_forward(x, W1, W2, topk_idx, gates, dtype) -> np.ndarray:
    """y [N, H] = sum_k gate * FFN_e(x), float64 with the layer's roundings."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gates, dtype=np.float64)
    y = np.zeros((x.shape[0], W2.shape[2]), dtype=np.float64)
    for e in range(W1.shape[0]):
        tok, kk = _slots_of(topk_idx, e)
        if len(tok) == 0:
            continue
        act = swiglu(x[tok] @ np.asarray(W1[e], dtype=np.float64), dtype)
        z = act @ np.asarray(W2[e], dtype=np.float64)
        np.add.at(y, tok, g[tok, kk][:, None] * z)
    return y


def dense_ffn_backward(x, W1, W2, topk_idx, d, dtype):
    """dx [N,H], dW1 [E,H,2H'], dW2 [E,H',H] (float64) from the gated upstream rows
    d [N*K, H]."""
    x = np.asarray(x, dtype=np.float64)
    d = np.asarray(d, dtype=np.float64)
    topk = np.asarray(topk_idx)
    K = topk.shape[1]
    dx = np.zeros_like(x)
    dW1 = np.zeros(W1.shape, dtype=np.float64)
    dW2 = np.zeros(W2.shape, dtype=np.float64)
    for e in range(W1.shape[0]):
        tok, kk = _slots_of(topk, e)
        if len(tok) == 0:
            continue
        w1 = np.asarray(W1[e], dtype=np.float64)
        w2 = np.asarray(W2[e], dtype=np.float64)
        de = d[tok * K + kk]
        h = x[tok] @ w1
        act = swiglu(h, dtype)
        dW2[e] = act.T @ de
        dh = swiglu_backward(round_to(h, dtype), de @ w2.T, dtype)
        np.add.at(dx, tok, dh @ w1.T)
        dW1[e] = x[tok].T @ dh
    return dx, dW1, dW2


# ----------------------------------------------------------------- plan-based pipeline

def pipeline_ffn_forward(x, W1, W2, topk_idx, gates, pl, R, S, E, K, B, dtype):
    """The library's order of steps in float64: prefetch both weights, permute,
    gate/up over the [E+B] view, SwiGLU, down over the view, gated combine.
    Returns (y, act) with act in buffer order [R*S*K, H']."""
    SK = S * K
    W1a = prefetch(W1, pl.replica_expert, E, B)
    W2a = prefetch(W2, pl.replica_expert, E, B)
    xp = permute(np.asarray(x, dtype=np.float64), pl.slot_map, K)
    h = segment_matmul(xp, W1a, pl.cu_seqlens, R, SK, E, B)
    act = swiglu(h, dtype)
    z = segment_matmul(act, W2a, pl.cu_seqlens, R, SK, E, B)
    return combine(z, pl.slot_map, gates, R * S, K), act


# ----------------------------------------------------------------- sampled checks

def slot_values(x_row, w1, w2, dtype):
    """(hs, act, z) of one slot: its token row x_row [H] through expert (w1, w2)."""
    h = np.asarray(x_row, dtype=np.float64) @ np.asarray(w1, dtype=np.float64)
    act = swiglu(h[None], dtype)[0]
    return round_to(h, dtype), act, act @ np.asarray(w2, dtype=np.float64)


def slot_backward(x_row, d_row, w1, w2, dtype):
    """(dh, dx contribution) of one slot: dh [2H'] and dh @ w1^T [H]."""
    w1 = np.asarray(w1, dtype=np.float64)
    h = np.asarray(x_row, dtype=np.float64) @ w1
    da = np.asarray(d_row, dtype=np.float64) @ np.asarray(w2, dtype=np.float64).T
    dh = swiglu_backward(round_to(h, dtype)[None], da[None], dtype)[0]
    return dh, dh @ w1.T


def wgrad_entries_ffn(x_rows, d_rows, w1, w2, hh, pp, dtype):
    """Entries of one expert's two weight gradients, computing only the columns
    they need (so a hot expert of thousands of slots stays cheap):

      dW1[hh[i], c] for c in the gate and up columns of intermediate columns pp
                    -> array [len(hh), 2, len(pp)] (index 1: 0 gate, 1 up)
      dW2[pp[i], :] -> array [len(pp), H]
    x_rows [n, H] and d_rows [n, H] are that expert's slots."""
    x_rows = np.asarray(x_rows, dtype=np.float64)
    d_rows = np.asarray(d_rows, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    Hp = w2.shape[0]
    gate, up = gate_up_columns(Hp)
    gcols, ucols = gate[pp], up[pp]
    hg = x_rows @ w1[:, gcols]                    # [n, len(pp)]
    hu = x_rows @ w1[:, ucols]
    act = round_to(silu(hg) * hu, dtype)
    dW2 = act.T @ d_rows                          # [len(pp), H]
    gs, us = round_to(hg, dtype), round_to(hu, dtype)
    da = d_rows @ w2[pp].T                        # [n, len(pp)]
    dg = round_to(da * us * silu_grad(gs), dtype)
    du = round_to(da * silu(gs), dtype)
    xs = x_rows[:, hh]
    dW1 = np.stack([xs.T @ dg, xs.T @ du], axis=1)
    return dW1, dW2
