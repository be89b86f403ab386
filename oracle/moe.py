"""Values of one expert projection around the plan.  TEST INFRASTRUCTURE.

The method reaches the plain dense result exactly: a duplicated expert holds the
same weights as its home copy, so where a slot is computed cannot change the
value [maestro "The memory contract": overflow experts read from home rows give
the same result, only slower].  The oracle therefore states the dense MoE
projection directly, in float64 over inputs already rounded to the layer dtype:

  forward    y[g]  = sum_k gate[g,k] * (x[g] @ W[e(g,k)])
  backward   d(u)  = bf16(fp32(gate[u]) * fp32(dy[g]))   (u = g*K + k; the one
                     rounding the gated permute of dY performs)
             dx[g] = sum_k d(gK+k) @ W[e]^T
             dW[e] = sum over slots u of e of outer(x[g], d(u))

and, separately, the plan-based pipeline the library runs (permute -> per-row
matmul on the [E+B,H,H'] view -> combine; replica gradients parked in an
[R,B,H,H'] buffer and folded home by reduce_grad), also in float64, so the
permutation semantics can be pinned against the dense result.

[maestro "The core idea": replicas are prefetched before expert compute, their
gradients return to the home ranks in backward; "The memory contract": fp32
[E+B,H,H'] grads with rows [E,E+B) backed by a separate reduce buffer viewed as
[R,B,H,H']; reduce_grad adds a rank's experts' slots from every rank into its
parameter grad and zeroes the consumed slots.]
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------- rounding

def bf16_round(a) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even; returned as float32.

    bfloat16 keeps the top 16 bits of an IEEE float32.  Adding 0x7FFF plus the
    lowest kept bit before truncation rounds to nearest with ties to even
    (finite inputs; NaN/Inf never occur in these layers).
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return (rounded & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)


# ----------------------------------------------------------------- dense form

def dense_forward(x, W, topk_idx, gates) -> np.ndarray:
    """y [N, H'] = sum_k gate * x @ W[e], float64, grouped by expert."""
    x = np.asarray(x, dtype=np.float64)
    topk = np.asarray(topk_idx)
    g = np.asarray(gates, dtype=np.float64)
    N, K = topk.shape
    y = np.zeros((N, W.shape[2]), dtype=np.float64)
    for e in range(W.shape[0]):
        tok, kk = np.nonzero(topk == e)
        if len(tok) == 0:
            continue
        contrib = x[tok] @ np.asarray(W[e], dtype=np.float64)
        np.add.at(y, tok, g[tok, kk][:, None] * contrib)
    return y


def gated_dy(dy, gates, dtype: str) -> np.ndarray:
    """d(u) = round_dtype(fp32(gate[u]) * fp32(dy[g])): [N*K, H'] float32 values."""
    dy = np.asarray(dy, dtype=np.float32)
    g = np.asarray(gates, dtype=np.float32)
    N, K = g.shape
    prod = (g[:, :, None] * dy[:, None, :]).astype(np.float32).reshape(N * K, -1)
    return bf16_round(prod) if dtype == "bf16" else prod


def dense_backward(x, W, topk_idx, d):
    """dx [N,H] and dW [E,H,H'] (float64) from the gated upstream rows d [N*K,H']."""
    x = np.asarray(x, dtype=np.float64)
    d = np.asarray(d, dtype=np.float64)
    topk = np.asarray(topk_idx)
    N, K = topk.shape
    E, H, Hp = W.shape
    dx = np.zeros((N, H), dtype=np.float64)
    dW = np.zeros((E, H, Hp), dtype=np.float64)
    for e in range(E):
        tok, kk = np.nonzero(topk == e)
        if len(tok) == 0:
            continue
        de = d[tok * K + kk]
        np.add.at(dx, tok, de @ np.asarray(W[e], dtype=np.float64).T)
        dW[e] = x[tok].T @ de
    return dx, dW


# ----------------------------------------------------------------- plan-based pipeline

def weight_row(W_all, q: int, i: int, E: int, B: int):
    """Rank q's row i of the [E+B,H,H'] view: home row i (i < E) or q's slot i-E,
    stored after the E home rows as row E + q*B + (i-E)."""
    return W_all[i] if i < E else W_all[E + q * B + (i - E)]


def prefetch(W, replica_expert, E: int, B: int):
    """W_all [E+R*B, H, H']: home rows plus each rank's prefetch slots filled with
    copies of the planned replica experts (unused slots stay zero)."""
    R = replica_expert.shape[0]
    W_all = np.zeros((E + R * B,) + W.shape[1:], dtype=W.dtype)
    W_all[:E] = W
    for q in range(R):
        for j in range(B):
            e = int(replica_expert[q, j])
            if e >= 0:
                W_all[E + q * B + j] = W[e]
    return W_all


def permute(rows, slot_map, K: int, per_slot: bool = False):
    """dst[slot_map[u]] = rows[u // K] (or rows[u] when per_slot)."""
    sm = np.asarray(slot_map)
    dst = np.zeros((len(sm), rows.shape[1]), dtype=rows.dtype)
    for u in range(len(sm)):
        dst[sm[u]] = rows[u] if per_slot else rows[u // K]
    return dst


def segment_matmul(a, W_all, cu_seqlens, R, SK, E, B, transpose_w=False):
    """c[q*SK + rows of (q,i)] = a[same rows] @ view_q(i) (or its transpose), float64."""
    cu = np.asarray(cu_seqlens)
    width = W_all.shape[1] if transpose_w else W_all.shape[2]
    c = np.zeros((a.shape[0], width), dtype=np.float64)
    for q in range(R):
        for i in range(E + B):
            lo, hi = q * SK + int(cu[q, i]), q * SK + int(cu[q, i + 1])
            if hi == lo:
                continue
            w = np.asarray(weight_row(W_all, q, i, E, B), dtype=np.float64)
            c[lo:hi] = np.asarray(a[lo:hi], dtype=np.float64) @ (w.T if transpose_w else w)
    return c


def combine(out, slot_map, gates, N: int, K: int):
    """y[g] = sum over k ascending of gate[g,k] * out[slot_map[g*K+k]] (gates None: 1)."""
    sm = np.asarray(slot_map)
    y = np.zeros((N, out.shape[1]), dtype=np.float64)
    for g in range(N):
        for k in range(K):
            w = 1.0 if gates is None else float(gates[g, k])
            y[g] += w * out[sm[g * K + k]]
    return y


def segment_wgrad(xp, dyp, cu_seqlens, R, SK, E, B, grad_home, reduce_buf):
    """Per non-empty row (q,i): D = xp_seg^T @ dyp_seg; i < E adds into grad_home[i],
    i >= E into reduce_buf[q, i-E] (the separate buffer behind rows [E,E+B))."""
    cu = np.asarray(cu_seqlens)
    for q in range(R):
        for i in range(E + B):
            lo, hi = q * SK + int(cu[q, i]), q * SK + int(cu[q, i + 1])
            if hi == lo:
                continue
            D = np.asarray(xp[lo:hi], dtype=np.float64).T @ np.asarray(dyp[lo:hi], dtype=np.float64)
            if i < E:
                grad_home[i] += D
            else:
                reduce_buf[q, i - E] += D


def reduce_grad(replica_expert, reduce_buf, grad_home):
    """For q ascending, then j ascending: grad_home[e] += reduce_buf[q,j] for the slot's
    expert e, then zero that slot (in place)."""
    R, B = replica_expert.shape
    for q in range(R):
        for j in range(B):
            e = int(replica_expert[q, j])
            if e >= 0:
                grad_home[e] += reduce_buf[q, j]
                reduce_buf[q, j] = 0


# ----------------------------------------------------------------- sampled checks

def dense_expert_outputs(x, W, topk_idx) -> np.ndarray:
    """out(u) = x[g] @ W[e(u)] for every slot u = g*K + k of the given tokens: [N*K, H'].

    ``W`` only needs ``W[e]`` for the experts these tokens use (it may fetch lazily)."""
    x = np.asarray(x, dtype=np.float64)
    topk = np.asarray(topk_idx)
    N, K = topk.shape
    Hp = W[int(topk.flat[0])].shape[1] if topk.size else 0
    out = np.zeros((N * K, Hp), dtype=np.float64)
    for e in np.unique(topk):
        tok, kk = np.nonzero(topk == e)
        out[tok * K + kk] = x[tok] @ np.asarray(W[int(e)], dtype=np.float64)
    return out


def wgrad_entries(x_rows, d_rows, hh, pp) -> np.ndarray:
    """Entries (hh[i], pp[j]) of sum over slots of one expert of outer(x[g], d(u)),
    given that expert's rows x_rows [n, H] and gated upstream rows d_rows [n, H']."""
    xs = np.asarray(x_rows, dtype=np.float64)[:, hh]
    ds = np.asarray(d_rows, dtype=np.float64)[:, pp]
    return xs.T @ ds
