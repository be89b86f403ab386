"""GPU parity where the other modules sample: the short-tail GEMM launch compared in
full, and whole output buffers at the full layer sizes.

* Layers large enough that the grouped GEMM treats segment tails (at most 128 rows)
  apart, but with a small hidden size, so the oracle computes every output: forward
  and backward of one projection and of the full expert FFN, element by element.
  DGRAD and the fused gate/up projection give the tails a launch of their own; a
  plain forward runs them in its 256-row tiles with the empty row group's
  wavefronts idle. The size (at least four rounds of full 256-row tiles over the
  compute units) is asserted, and so are the tails themselves.
* Full-size layers, outputs poisoned with NaN before the call: every element of
  every output buffer is finite afterwards, and the first and last slot of every
  non-empty segment, plus the first slot of the segment's last 256-row tile (a tail
  tile where the tails are split off), equal the oracle's value over every column.
  The weight gradients are checked at one entry inside every 256 x 256 gradient
  tile (and the last row and column) of every expert.

Tolerances as elsewhere: max abs error <= 1e-2 * RMS(reference) for bfloat16 layers
[the hot path's rows: ai-maestro.online "Moonshot AI open-sources MoonEP", sections
"The core idea: dynamic redundant experts" (every rank's fixed S*K buffer) and
"The memory contract" (rows selected by cu_seqlens)].
"""
import numpy as np
import pytest
import torch

from oracle import ffn as FF
from oracle import moe as M
from oracle import plan as P
from redundant_expert_balancing_amd.ffn import MoEFFN
from redundant_expert_balancing_amd.layer import MoEProjection
from redundant_expert_balancing_amd.synth import CONFIGS, make_dense, make_routing

from gpu_helpers import assert_stored_close, rel_err, say, small_cfg, tolerance

pytestmark = pytest.mark.gpu

TILE_M = 256      # rows of a full M-tile of the bf16 grouped GEMM
TAIL_ROWS = 128   # a segment's last tile with at most this many rows is a short tail


def _host(t):
    return t.float().cpu().numpy()


def _tails_split(cfg, ncols) -> bool:
    """Whether the GEMM over R*S*K rows and `ncols` output columns is large enough to
    treat its tails apart (DGRAD and the fused gate/up projection launch them on their
    own): at least four rounds of full 256 x 256 tiles over the device's compute units."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return cfg.R * cfg.S * cfg.K // TILE_M * -(-ncols // TILE_M) >= 4 * cus


def _n_short_tails(cu) -> int:
    n = 0
    for q in range(cu.shape[0]):
        for i in range(cu.shape[1] - 1):
            m = int(cu[q, i + 1]) - int(cu[q, i])
            if m > 0 and m - (m - 1) // TILE_M * TILE_M <= TAIL_ROWS:
                n += 1
    return n


def _segment_end_rows(cu, SK):
    """Buffer rows of the first and last slot of every non-empty segment and the first
    slot of its last 256-row tile."""
    rows = set()
    for q in range(cu.shape[0]):
        for i in range(cu.shape[1] - 1):
            lo, hi = int(cu[q, i]), int(cu[q, i + 1])
            if hi > lo:
                last = lo + (hi - lo - 1) // TILE_M * TILE_M
                rows.update((q * SK + lo, q * SK + last, q * SK + hi - 1))
    return np.array(sorted(rows), dtype=np.int64)


def _all_finite(**bufs):
    for name, t in bufs.items():
        bad = int((~torch.isfinite(t)).sum())
        assert bad == 0, f"{name}: {bad} of {t.numel()} elements not finite (unwritten)"


# ------------------------------------------------------------ tail-launch shapes

TAIL_CFG = dict(R=8, S=3072, E=128, K=8, H=384, Hp=320)


def test_tail_launch_projection_full_compare():
    cfg = small_cfg(name="tails_projection", **TAIL_CFG)
    say("tail launch projection", TAIL_CFG)
    assert _tails_split(cfg, cfg.Hp) and _tails_split(cfg, cfg.H)
    r = make_routing(cfg, 3.0, alpha=1.0)
    d = make_dense(cfg, "cuda", 0, w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEProjection(cfg, "cuda", backward=True, w_all=d["W"])
    topk, gates = torch.from_numpy(r.topk_idx).cuda(), torch.from_numpy(r.gates).cuda()
    layer.grad_home.zero_()
    for t in (layer.out, layer.y, layer.dxp, layer.dx):
        t.fill_(float("nan"))
    y = layer.forward(topk, d["x"], gates)
    dx = layer.backward(d["dy"], gates)
    torch.cuda.synchronize()
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert np.array_equal(layer.cu_seqlens.cpu().numpy(), pl.cu_seqlens)
    assert np.array_equal(layer.slot_map.cpu().numpy(), pl.slot_map)
    tails = _n_short_tails(pl.cu_seqlens)
    say("short tails", tails, "replicas", pl.n_replicas)
    assert tails >= 16 and pl.n_replicas > 0
    x_h, W_h, dy_h = _host(d["x"]), _host(d["W"][:cfg.E]), _host(d["dy"])
    out_ref = M.dense_expert_outputs(x_h, W_h, r.topk_idx)
    assert rel_err(_host(layer.out)[pl.slot_map], out_ref) <= tolerance(cfg)
    assert rel_err(_host(y), M.dense_forward(x_h, W_h, r.topk_idx, r.gates)) <= tolerance(cfg)
    dd = M.gated_dy(dy_h, r.gates, cfg.dtype)
    dx_ref, dW_ref = M.dense_backward(x_h, W_h, r.topk_idx, dd)
    # dgrad of every slot before the unpermute: d(u) @ W[e]^T
    dxp_ref = np.zeros((cfg.N * cfg.K, cfg.H))
    for e in range(cfg.E):
        tok, kk = np.nonzero(r.topk_idx == e)
        u = tok * cfg.K + kk
        dxp_ref[u] = dd[u].astype(np.float64) @ W_h[e].astype(np.float64).T
    assert rel_err(_host(layer.dxp)[pl.slot_map], dxp_ref) <= tolerance(cfg)
    e_dx = rel_err(_host(dx), dx_ref)
    e_dw = rel_err(_host(layer.grad_home), dW_ref)
    say("tail launch projection: dx", e_dx, "dW", e_dw)
    assert max(e_dx, e_dw) <= tolerance(cfg)
    assert int(torch.count_nonzero(layer.reduce_buf)) == 0


def test_tail_launch_ffn_full_compare():
    cfg = small_cfg(name="tails_ffn", **TAIL_CFG)
    say("tail launch ffn", TAIL_CFG)
    # gate/up (2H' columns), down (H columns) and the W1 dgrad (H columns)
    assert _tails_split(cfg, 2 * cfg.Hp) and _tails_split(cfg, cfg.H)
    r = make_routing(cfg, 3.0, alpha=1.0)
    d = make_dense(cfg, "cuda", 0, which=("x", "W1", "W2", "dyH"), w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEFFN(cfg, "cuda", backward=True, w1_all=d["W1"], w2_all=d["W2"])
    topk, gates = torch.from_numpy(r.topk_idx).cuda(), torch.from_numpy(r.gates).cuda()
    for t in (layer.act, layer.hs, layer.dh):
        t.view(torch.int16).fill_(-1)
    for t in (layer.z, layer.y, layer.da, layer.dxp, layer.dx):
        t.fill_(float("nan"))
    y = layer.forward(topk, d["x"], gates)
    dx = layer.backward(d["dyH"], gates)
    torch.cuda.synchronize()
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert np.array_equal(layer.slot_map.cpu().numpy(), pl.slot_map)
    assert _n_short_tails(pl.cu_seqlens) >= 16
    x_h, dy_h = _host(d["x"]), _host(d["dyH"])
    W1, W2 = _host(d["W1"][:cfg.E]), _host(d["W2"][:cfg.E])
    N, K = cfg.N, cfg.K
    act_ref = np.zeros((N * K, cfg.Hp))
    hs_ref = np.zeros((N * K, 2 * cfg.Hp))
    z_ref = np.zeros((N * K, cfg.H))
    for e in range(cfg.E):
        tok, kk = np.nonzero(r.topk_idx == e)
        h = x_h[tok].astype(np.float64) @ W1[e].astype(np.float64)
        a = FF.swiglu(h, cfg.dtype)
        act_ref[tok * K + kk] = a
        hs_ref[tok * K + kk] = FF.round_to(h, cfg.dtype)
        z_ref[tok * K + kk] = a @ W2[e].astype(np.float64)
    assert_stored_close(_host(layer.act)[pl.slot_map], act_ref, cfg.dtype, "act")
    assert_stored_close(_host(layer.hs)[pl.slot_map], hs_ref, cfg.dtype, "hs")
    assert rel_err(_host(layer.z)[pl.slot_map], z_ref) <= tolerance(cfg)
    e_y = rel_err(_host(y), FF.dense_ffn_forward(x_h, W1, W2, r.topk_idx, r.gates, cfg.dtype))
    dd = M.gated_dy(dy_h, r.gates, cfg.dtype)
    dx_ref, dW1, dW2 = FF.dense_ffn_backward(x_h, W1, W2, r.topk_idx, dd, cfg.dtype)
    e_dx = rel_err(_host(dx), dx_ref)
    e1 = rel_err(_host(layer.grad1), dW1)
    e2 = rel_err(_host(layer.grad2), dW2)
    say("tail launch ffn: y", e_y, "dx", e_dx, "dW1", e1, "dW2", e2)
    assert max(e_y, e_dx, e1, e2) <= tolerance(cfg)
    assert int(torch.count_nonzero(layer.red1)) == 0 and int(torch.count_nonzero(layer.red2)) == 0


# ------------------------------------------------------------ full sizes

def _rows_oracle(cfg, topk, src, rows, w_dev, a_rows, transpose_w=False):
    """Oracle value of buffer rows `rows`: a_rows[i] @ W[e] (or W[e]^T) for the expert e
    of the slot held there, fetching one expert's weights at a time."""
    u = src[rows]
    e_of = topk.reshape(-1)[u]
    width = w_dev.shape[1] if transpose_w else w_dev.shape[2]
    ref = np.zeros((len(rows), width))
    for e in np.unique(e_of):
        sel = np.nonzero(e_of == e)[0]
        w = w_dev[int(e)].float().cpu().numpy().astype(np.float64)
        ref[sel] = a_rows[sel].astype(np.float64) @ (w.T if transpose_w else w)
    return ref


@pytest.mark.parametrize("key", [("bench_shape", 20.0), ("infer_overflow", 10.0)],
                         ids=lambda k: f"{k[0]}-{k[1]}")
def test_forward_full_size_whole_buffers_and_segment_ends(key):
    name, target = key
    cfg = CONFIGS[name]
    say("forward whole buffers", name, target)
    r = make_routing(cfg, target)
    d = make_dense(cfg, "cuda", 0, which=("x", "W"), w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEProjection(cfg, "cuda", w_all=d["W"])
    topk, gates = torch.from_numpy(r.topk_idx).cuda(), torch.from_numpy(r.gates).cuda()
    layer.out.fill_(float("nan"))
    layer.y.fill_(float("nan"))
    layer.forward(topk, d["x"], gates)
    torch.cuda.synchronize()
    _all_finite(out=layer.out, y=layer.y)
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert np.array_equal(layer.cu_seqlens.cpu().numpy(), pl.cu_seqlens)
    rows = _segment_end_rows(pl.cu_seqlens, cfg.SK)
    nseg = int((np.diff(pl.cu_seqlens, axis=1) > 0).sum())
    u = pl.src_index[rows]
    x_rows = _host(d["x"][torch.from_numpy(u // cfg.K).long().cuda()])
    ref = _rows_oracle(cfg, r.topk_idx, pl.src_index, rows, d["W"], x_rows)
    got = _host(layer.out[torch.from_numpy(rows).cuda()])
    err = rel_err(got, ref)
    say("forward whole buffers", name, nseg, "segments,", len(rows), "rows, max err / RMS", err,
        "short tails", _n_short_tails(pl.cu_seqlens))
    assert err <= tolerance(cfg)


def test_backward_full_size_whole_buffers_and_segment_ends():
    cfg = CONFIGS["train_backward"]
    say("backward whole buffers", cfg.name)
    r = make_routing(cfg, 15.0)
    d = make_dense(cfg, "cuda", 0, which=("x", "W", "dy"), w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEProjection(cfg, "cuda", backward=True, w_all=d["W"])
    topk, gates = torch.from_numpy(r.topk_idx).cuda(), torch.from_numpy(r.gates).cuda()
    layer.grad_home.zero_()
    for t in (layer.out, layer.y, layer.dxp, layer.dx):
        t.fill_(float("nan"))
    layer.forward(topk, d["x"], gates)
    layer.backward(d["dy"], gates)
    torch.cuda.synchronize()
    _all_finite(out=layer.out, y=layer.y, dxp=layer.dxp, dx=layer.dx, grad_home=layer.grad_home)
    assert int(torch.count_nonzero(layer.reduce_buf)) == 0
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert np.array_equal(layer.cu_seqlens.cpu().numpy(), pl.cu_seqlens)
    K = cfg.K
    # dgrad rows before the unpermute: d(u) @ W[e]^T at every segment's ends
    rows = _segment_end_rows(pl.cu_seqlens, cfg.SK)
    u = pl.src_index[rows]
    g_dev = torch.from_numpy(u // K).long().cuda()
    d_rows = M.gated_dy(_host(d["dy"][g_dev]), r.gates[u // K], cfg.dtype)
    d_rows = d_rows[np.arange(len(u)) * K + u % K]
    ref = _rows_oracle(cfg, r.topk_idx, pl.src_index, rows, d["W"], d_rows, transpose_w=True)
    err = rel_err(_host(layer.dxp[torch.from_numpy(rows).cuda()]), ref)
    say("dgrad segment ends", len(rows), "rows, max err / RMS", err)
    assert err <= tolerance(cfg)
    # weight gradients: one entry inside every 256 x 256 tile of every expert, plus the
    # last row and column (home segments and replicas folded by reduce_grad)
    rng = np.random.default_rng(5)
    hh = np.array([t + int(rng.integers(min(TILE_M, cfg.H - t))) for t in range(0, cfg.H, TILE_M)]
                  + [cfg.H - 1])
    pp = np.array([t + int(rng.integers(min(TILE_M, cfg.Hp - t))) for t in range(0, cfg.Hp, TILE_M)]
                  + [cfg.Hp - 1])
    hh_d, pp_d = torch.from_numpy(hh).cuda(), torch.from_numpy(pp).cuda()
    got_all, ref_all = [], []
    for ex in range(cfg.E):
        tok, kk = np.nonzero(r.topk_idx == ex)
        got_all.append(_host(layer.grad_home[ex][hh_d][:, pp_d]))
        if len(tok) == 0:
            ref_all.append(np.zeros((len(hh), len(pp))))
            continue
        t_dev = torch.from_numpy(tok).cuda()
        x_rows = _host(d["x"][t_dev][:, hh_d])
        dg = M.gated_dy(_host(d["dy"][t_dev][:, pp_d]), r.gates[tok, kk][:, None], cfg.dtype)
        ref_all.append(M.wgrad_entries(x_rows, dg, np.arange(len(hh)), np.arange(len(pp))))
    err = rel_err(np.stack(got_all), np.stack(ref_all))
    say("wgrad tile entries", cfg.E, "experts x", len(hh) * len(pp), "entries, max err / RMS", err)
    assert err <= tolerance(cfg)


@pytest.mark.parametrize("key", [("bench_shape", 20.0), ("infer_overflow", 10.0)],
                         ids=lambda k: f"{k[0]}-{k[1]}")
def test_ffn_forward_full_size_whole_buffers(key):
    name, target = key
    cfg = CONFIGS[name]
    say("ffn forward whole buffers", name, target)
    r = make_routing(cfg, target)
    d = make_dense(cfg, "cuda", 0, which=("x", "W1", "W2"), w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEFFN(cfg, "cuda", backward=False, w1_all=d["W1"], w2_all=d["W2"])
    topk, gates = torch.from_numpy(r.topk_idx).cuda(), torch.from_numpy(r.gates).cuda()
    layer.act.view(torch.int16).fill_(-1)
    layer.z.fill_(float("nan"))
    layer.y.fill_(float("nan"))
    layer.forward(topk, d["x"], gates)
    torch.cuda.synchronize()
    _all_finite(act=layer.act, z=layer.z, y=layer.y)
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert np.array_equal(layer.cu_seqlens.cpu().numpy(), pl.cu_seqlens)
    # act and z of the segment ends of a spread of experts, the whole slot in the oracle
    flat = r.topk_idx.reshape(-1)
    rows = _segment_end_rows(pl.cu_seqlens, cfg.SK)
    u = pl.src_index[rows]
    e_of = flat[u]
    keep = np.isin(e_of, np.unique(e_of)[::8])
    rows, u, e_of = rows[keep], u[keep], e_of[keep]
    x_rows = _host(d["x"][torch.from_numpy(u // cfg.K).long().cuda()])
    act_ref = np.zeros((len(rows), cfg.Hp))
    z_ref = np.zeros((len(rows), cfg.H))
    for e in np.unique(e_of):
        w1 = _host(d["W1"][int(e)]).astype(np.float64)
        w2 = _host(d["W2"][int(e)]).astype(np.float64)
        for i in np.nonzero(e_of == e)[0]:
            _, act_ref[i], z_ref[i] = FF.slot_values(x_rows[i], w1, w2, cfg.dtype)
    rows_d = torch.from_numpy(rows).cuda()
    assert_stored_close(_host(layer.act[rows_d]), act_ref, cfg.dtype, "act")
    err = rel_err(_host(layer.z[rows_d]), z_ref)
    say("ffn segment ends", len(np.unique(e_of)), "experts,", len(rows), "rows, z max err / RMS", err)
    assert err <= tolerance(cfg)


def test_ffn_backward_full_size_whole_buffers():
    cfg = CONFIGS["train_backward"]
    say("ffn backward whole buffers", cfg.name)
    r = make_routing(cfg, 15.0)
    d = make_dense(cfg, "cuda", 0, which=("x", "W1", "W2", "dyH"), w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEFFN(cfg, "cuda", backward=True, w1_all=d["W1"], w2_all=d["W2"])
    topk, gates = torch.from_numpy(r.topk_idx).cuda(), torch.from_numpy(r.gates).cuda()
    for t in (layer.act, layer.hs, layer.dh, layer.dyp):
        t.view(torch.int16).fill_(-1)
    for t in (layer.z, layer.y, layer.da, layer.dxp, layer.dx):
        t.fill_(float("nan"))
    layer.forward(topk, d["x"], gates)
    layer.backward(d["dyH"], gates)
    torch.cuda.synchronize()
    _all_finite(act=layer.act, hs=layer.hs, z=layer.z, y=layer.y, dyp=layer.dyp, da=layer.da,
                dh=layer.dh, dxp=layer.dxp, dx=layer.dx, grad1=layer.grad1, grad2=layer.grad2)
    assert int(torch.count_nonzero(layer.red1)) == 0 and int(torch.count_nonzero(layer.red2)) == 0
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert np.array_equal(layer.cu_seqlens.cpu().numpy(), pl.cu_seqlens)
    # the W1 dgrad rows (before the unpermute) at every segment's ends: the slot's whole
    # backward chain in the oracle, dh(u) @ W1[e]^T
    K = cfg.K
    flat = r.topk_idx.reshape(-1)
    rows = _segment_end_rows(pl.cu_seqlens, cfg.SK)
    u = pl.src_index[rows]
    e_of = flat[u]
    g_dev = torch.from_numpy(u // K).long().cuda()
    x_rows = _host(d["x"][g_dev])
    d_rows = M.gated_dy(_host(d["dyH"][g_dev]), r.gates[u // K], cfg.dtype)
    d_rows = d_rows[np.arange(len(u)) * K + u % K]
    ref = np.zeros((len(rows), cfg.H))
    for e in np.unique(e_of):
        w1 = _host(d["W1"][int(e)]).astype(np.float64)
        w2 = _host(d["W2"][int(e)]).astype(np.float64)
        for i in np.nonzero(e_of == e)[0]:
            ref[i] = FF.slot_backward(x_rows[i], d_rows[i], w1, w2, cfg.dtype)[1]
    err = rel_err(_host(layer.dxp[torch.from_numpy(rows).cuda()]), ref)
    say("ffn W1 dgrad segment ends", len(rows), "rows, max err / RMS", err)
    assert err <= tolerance(cfg)
