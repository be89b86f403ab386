"""GPU value parity of the full expert FFN on the plan: gate/up grouped GEMM with
the SwiGLU (fused into its epilogue, and as a separate pass), down grouped GEMM,
combine, and the backward (gated dispatch of dY, dgrad and wgrad of W2, SwiGLU
backward, dgrad and wgrad of W1, unpermute, reduce_grad of both weights) against
the float64 oracle (oracle/ffn.py) on the same inputs.

Small layers are compared element by element everywhere, full-size layers on
sampled tokens and experts. The fused and the unfused gate/up paths must agree
bit for bit (same float32 accumulators, same activation function). Tolerances:
max abs error <= 1e-2 * RMS(reference) for bf16 layers, <= 1e-5 * RMS for fp32;
the standalone SwiGLU kernels within one bfloat16 rounding step (bf16) or a few
float32 ulps (fp32) of the oracle, element by element.
"""
import numpy as np
import pytest
import torch

from oracle import ffn as FF
from oracle import moe as M
from oracle import plan as P
from redundant_expert_balancing_amd import _lib as L
from redundant_expert_balancing_amd.ffn import MoEFFN
from redundant_expert_balancing_amd.synth import CONFIGS, make_dense, make_routing

from gpu_helpers import assert_plan_equal, assert_stored_close, rel_err, say, small_cfg, tolerance

pytestmark = pytest.mark.gpu


def _host(t):
    return t.float().cpu().numpy()


def _setup(cfg, target, backward=False, alpha=None, seed=0, fused=True):
    r = make_routing(cfg, target, seed=seed, alpha=alpha)
    which = ("x", "W1", "W2", "dyH") if backward else ("x", "W1", "W2")
    d = make_dense(cfg, "cuda", seed, which=which, w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEFFN(cfg, "cuda", backward=backward, w1_all=d["W1"], w2_all=d["W2"], fused=fused)
    topk = torch.from_numpy(r.topk_idx).cuda()
    gates = torch.from_numpy(r.gates).cuda()
    return r, layer, d, topk, gates


def _poison(layer):
    for t in (layer.xp, layer.act):
        t.view(torch.int16).fill_(-1)
    layer.z.fill_(float("nan"))
    layer.y.fill_(float("nan"))
    if layer.hs is not None:
        layer.hs.view(torch.int16).fill_(-1)


def _by_expert(slots, topk, K):
    """{expert: [slot u, ...]} for the given flat slot ids."""
    out = {}
    for u in slots:
        out.setdefault(int(topk[u // K, u % K]), []).append(int(u))
    return out


def _slot_oracle(d, cfg, topk, slots):
    """Per slot u: (hs, act, z) from the oracle, fetching each expert's W1 and W2
    once (host memory stays at one expert's weights)."""
    res = {}
    for e, us in _by_expert(slots, topk, cfg.K).items():
        w1, w2 = _host(d["W1"][e]), _host(d["W2"][e])
        xs = _host(d["x"][torch.tensor([u // cfg.K for u in us], device="cuda")])
        for i, u in enumerate(us):
            res[u] = FF.slot_values(xs[i], w1, w2, cfg.dtype)
    return res


@pytest.mark.parametrize("name", ["tiny_fp32_train", "bf16_train_mild"])
def test_ffn_forward_full_compare(name):
    cfg = CONFIGS[name]
    say("ffn forward full", name)
    r, layer, d, topk, gates = _setup(cfg, cfg.maxvio[0], backward=True)
    _poison(layer)
    w1_home, w2_home = d["W1"][:cfg.E].clone(), d["W2"][:cfg.E].clone()
    y = layer.forward(topk, d["x"], gates)
    torch.cuda.synchronize()
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert_plan_equal({"cu_seqlens": layer.cu_seqlens.cpu().numpy(),
                       "replica_expert": layer.replica_expert[:, :cfg.B].cpu().numpy(),
                       "slot_map": layer.slot_map.cpu().numpy(),
                       "src_index": layer.src_index.cpu().numpy()}, pl)
    assert torch.equal(d["W1"][:cfg.E], w1_home) and torch.equal(d["W2"][:cfg.E], w2_home)
    for q in range(cfg.R):
        for j in range(cfg.B):
            e = int(pl.replica_expert[q, j])
            if e >= 0:
                assert torch.equal(layer.w1_all[cfg.E + q * cfg.B + j], w1_home[e])
                assert torch.equal(layer.w2_all[cfg.E + q * cfg.B + j], w2_home[e])
    x_h, W1, W2 = _host(d["x"]), _host(w1_home), _host(w2_home)
    # the activation of every slot, in buffer order
    N, K = cfg.R * cfg.S, cfg.K
    act_ref = np.zeros((N * K, cfg.Hp))
    hs_ref = np.zeros((N * K, 2 * cfg.Hp))
    for e in range(cfg.E):
        tok, kk = np.nonzero(r.topk_idx == e)
        h = x_h[tok].astype(np.float64) @ W1[e]
        act_ref[tok * K + kk] = FF.swiglu(h, cfg.dtype)
        hs_ref[tok * K + kk] = FF.round_to(h, cfg.dtype)
    assert_stored_close(_host(layer.act)[pl.slot_map], act_ref, cfg.dtype, "act")
    assert_stored_close(_host(layer.hs)[pl.slot_map], hs_ref, cfg.dtype, "hs")
    y_ref = FF.dense_ffn_forward(x_h, W1, W2, r.topk_idx, r.gates, cfg.dtype)
    err = rel_err(_host(y), y_ref)
    say("ffn forward full", name, "max err / RMS", err)
    assert err <= tolerance(cfg)
    # the unfused path (GEMM to float32 h, then the SwiGLU pass) gives the same bits
    act_f, hs_f, y_f = layer.act.clone(), layer.hs.clone(), layer.y.clone()
    layer.fused = False
    layer.h = torch.empty((N * K, 2 * cfg.Hp), dtype=torch.float32, device="cuda")
    _poison(layer)
    layer.forward(topk, d["x"], gates)
    torch.cuda.synchronize()
    assert torch.equal(layer.act, act_f) and torch.equal(layer.hs, hs_f)
    assert torch.equal(layer.y, y_f)


@pytest.mark.parametrize("H,Hp", [(64, 96), (128, 32), (192, 160)])
def test_fused_swiglu_gemm_partial_tiles_match_unfused(H, Hp):
    """Intermediate sizes whose 2H' columns end inside a 256-column tile (whole
    wavefronts of the tile are past the end): fused == GEMM + SwiGLU, bit for bit."""
    cfg = small_cfg(name=f"fused_{H}_{Hp}", R=2, S=45, E=8, K=2, H=H, Hp=2 * Hp)
    say("fused partial tiles", H, Hp)
    r = make_routing(cfg, 1.0, alpha=1.5)
    g = torch.Generator(device="cuda").manual_seed(7)
    rows = cfg.R * cfg.S * cfg.K
    W = cfg.E + cfg.R * cfg.B
    x = torch.randn((cfg.N, H), generator=g, device="cuda").to(torch.bfloat16)
    w1 = (torch.randn((W, H, 2 * Hp), generator=g, device="cuda") * H ** -0.5).to(torch.bfloat16)
    shp = L.Shape(cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, H, Hp, L.TRAIN, L.BF16)
    up = L.Shape(cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, H, 2 * Hp, L.TRAIN, L.BF16)
    i32 = dict(dtype=torch.int32, device="cuda")
    cu = torch.empty((cfg.R, cfg.E + cfg.B + 1), **i32)
    rep = torch.empty((cfg.R, cfg.B), **i32)
    sm = torch.empty((rows,), **i32)
    si = torch.empty((rows,), **i32)
    ws = torch.empty((L.moonep_workspace_bytes(up) // 4,), **i32)
    L.moonep_workspace_init(up, ws)
    L.moonep_plan(up, torch.from_numpy(r.topk_idx).cuda(), cu, rep, sm, si, ws)
    L.moonep_prefetch_weight(up, rep, w1)
    xp = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    L.moonep_dispatch(up, H, x, sm, None, xp)
    act_a = torch.full((rows, Hp), float("nan"), dtype=torch.bfloat16, device="cuda")
    hs_a = torch.full((rows, 2 * Hp), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.moonep_grouped_gemm_swiglu(shp, xp, w1, cu, act_a, hs_a, ws)
    h = torch.full((rows, 2 * Hp), float("nan"), device="cuda")
    L.moonep_grouped_gemm(up, L.FWD, xp, w1, cu, h, None, None, ws)
    act_b = torch.full_like(act_a, float("nan"))
    hs_b = torch.full_like(hs_a, float("nan"))
    L.moonep_swiglu(shp, h, act_b, hs_b)
    torch.cuda.synchronize()
    assert torch.equal(act_a, act_b) and torch.equal(hs_a, hs_b)
    assert torch.equal(hs_b, h.to(torch.bfloat16))
    # and the values are the oracle's
    topk = r.topk_idx
    src = si.cpu().numpy()
    hh = h.cpu().numpy().astype(np.float64)
    xh, w1h = _host(x), _host(w1)
    for i in np.random.default_rng(0).choice(rows, 40, replace=False):
        u = int(src[i])
        e = int(topk[u // cfg.K, u % cfg.K])
        want = FF.swiglu((xh[u // cfg.K].astype(np.float64) @ w1h[e])[None], "bf16")[0]
        assert_stored_close(_host(act_a[i]), want, "bf16", f"act row {i}")
        assert np.allclose(hh[i], xh[u // cfg.K].astype(np.float64) @ w1h[e], rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_swiglu_kernels_elementwise(dtype):
    """moonep_swiglu / moonep_swiglu_backward against the oracle element by element
    on values spanning the sigmoid's range (|v| up to 30)."""
    say("swiglu kernels", dtype)
    R, S, K, Hp = 2, 33, 2, 96
    rows = R * S * K
    shp = L.Shape(R, S, 8, K, 4, 64, Hp, L.TRAIN, L.BF16 if dtype == "bf16" else L.FP32)
    g = torch.Generator(device="cuda").manual_seed(3)
    h = torch.randn((rows, 2 * Hp), generator=g, device="cuda") * 4.0
    h[0, :32] = torch.linspace(-30, 30, 32, device="cuda")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    act = torch.empty((rows, Hp), dtype=dt, device="cuda")
    hs = torch.empty((rows, 2 * Hp), dtype=dt, device="cuda")
    L.moonep_swiglu(shp, h, act, hs)
    da = torch.randn((rows, Hp), generator=g, device="cuda")
    dh = torch.empty((rows, 2 * Hp), dtype=dt, device="cuda")
    L.moonep_swiglu_backward(shp, hs, da, dh)
    torch.cuda.synchronize()
    hn = h.cpu().numpy().astype(np.float64)
    act_ref = FF.swiglu(hn, dtype)
    hs_n = _host(hs).astype(np.float64)
    assert np.array_equal(hs_n, FF.round_to(hn, dtype))
    da_n = da.cpu().numpy().astype(np.float64)
    dh_ref = FF.swiglu_backward(hs_n, da_n, dtype)
    # float32 evaluation error, bounded by the magnitude of the terms it sums
    # (dgate = da*u*(s + g*s*(1-s)) cancels near g = -1.28)
    gate, up = FF.gate_up_columns(Hp)
    gv, uv = hs_n[:, gate], hs_n[:, up]
    sg = FF.sigmoid(gv)
    terms = np.zeros_like(hs_n)
    terms[:, gate] = np.abs(da_n * uv) * (sg + np.abs(gv) * sg * (1 - sg))
    terms[:, up] = np.abs(da_n * gv) * sg
    # one rounding step of the stored type (bf16: 2^-7 of the value at most) plus
    # a few float32 ulps of the terms
    step = 2.0 ** -7 if dtype == "bf16" else 2e-6
    assert np.all(np.abs(_host(act) - act_ref) <= step * np.abs(act_ref) + 1e-30)
    assert np.all(np.abs(_host(dh) - dh_ref) <= step * np.abs(dh_ref) + 2.0 ** -21 * terms + 1e-30)


def _ffn_backward_check(cfg, target, alpha=None, full=False):
    say("ffn backward", cfg.name, target, "full" if full else "sampled")
    r, layer, d, topk, gates = _setup(cfg, target, backward=True, alpha=alpha)
    g0 = torch.Generator(device="cuda").manual_seed(123)
    init1 = torch.randn(layer.grad1.shape, generator=g0, device="cuda")
    init2 = torch.randn(layer.grad2.shape, generator=g0, device="cuda")
    layer.grad1.copy_(init1)          # grads accumulate (+=) into whatever is there
    layer.grad2.copy_(init2)
    layer.forward(topk, d["x"], gates)
    for t in (layer.dyp, layer.dh):
        t.view(torch.int16).fill_(-1)
    for t in (layer.da, layer.dxp, layer.dx):
        t.fill_(float("nan"))
    dx = layer.backward(d["dyH"], gates)
    torch.cuda.synchronize()
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert pl.n_replicas > 0
    assert int(torch.count_nonzero(layer.red1)) == 0
    assert int(torch.count_nonzero(layer.red2)) == 0
    sm = layer.slot_map.long()
    u = torch.arange(sm.numel(), device="cuda")
    want = (gates.reshape(-1)[u][:, None] * d["dyH"].float()[u // cfg.K]).to(layer.dtype)
    assert torch.equal(layer.dyp[sm], want)
    N, K = cfg.R * cfg.S, cfg.K
    tol = tolerance(cfg)
    if full:
        x_h, dy_h = _host(d["x"]), _host(d["dyH"])
        W1, W2 = _host(d["W1"][:cfg.E]), _host(d["W2"][:cfg.E])
        dd = M.gated_dy(dy_h, r.gates, cfg.dtype)
        dx_ref, dW1, dW2 = FF.dense_ffn_backward(x_h, W1, W2, r.topk_idx, dd, cfg.dtype)
        e_dx = rel_err(_host(dx), dx_ref)
        e1 = float(np.abs(_host(layer.grad1) - _host(init1) - dW1).max() / np.sqrt(np.mean(dW1 ** 2)))
        e2 = float(np.abs(_host(layer.grad2) - _host(init2) - dW2).max() / np.sqrt(np.mean(dW2 ** 2)))
        say("ffn backward full: dx", e_dx, "dW1", e1, "dW2", e2)
        assert max(e_dx, e1, e2) <= tol
        return
    # sampled tokens: dx[g] = sum_k dh(u) @ W1[e]^T
    rng = np.random.default_rng(2)
    toks = np.sort(rng.choice(N, 12, replace=False))
    slots = (toks[:, None] * K + np.arange(K)[None, :]).ravel()
    dy_s = _host(d["dyH"][torch.from_numpy(toks).cuda()])
    dd = M.gated_dy(dy_s, r.gates[toks], cfg.dtype)           # [len(toks)*K, H]
    dx_ref = np.zeros((len(toks), cfg.H))
    row_of = {int(g): i for i, g in enumerate(toks)}
    for e, us in _by_expert(slots, r.topk_idx, K).items():
        w1, w2 = _host(d["W1"][e]), _host(d["W2"][e])
        xs = _host(d["x"][torch.tensor([u // K for u in us], device="cuda")])
        for i, uu in enumerate(us):
            ti = row_of[uu // K]
            dx_ref[ti] += FF.slot_backward(xs[i], dd[ti * K + uu % K], w1, w2, cfg.dtype)[1]
    e_dx = rel_err(_host(dx[torch.from_numpy(toks).cuda()]), dx_ref)
    say("ffn backward sampled dx err", e_dx)
    assert e_dx <= tol
    # weight gradients of replicated experts (folded home) and two others, on
    # sampled rows and columns
    experts = sorted(set(int(x) for x in pl.replica_expert.ravel() if x >= 0))[:3]
    experts += [int(x) for x in rng.choice(cfg.E, 2, replace=False) if x not in experts]
    hh = np.sort(rng.choice(cfg.H, 16, replace=False))
    pp = np.sort(rng.choice(cfg.Hp, 16, replace=False))
    gate, up = FF.gate_up_columns(cfg.Hp)
    hh_d, pp_d = torch.from_numpy(hh).cuda(), torch.from_numpy(pp).cuda()
    for ex in experts:
        tok, kk = np.nonzero(r.topk_idx == ex)
        if len(tok) == 0:
            continue
        t_dev = torch.from_numpy(tok).cuda()
        x_rows = _host(d["x"][t_dev])
        d_rows = M.gated_dy(_host(d["dyH"][t_dev]), r.gates[tok, kk][:, None], cfg.dtype)
        dW1, dW2 = FF.wgrad_entries_ffn(x_rows, d_rows, _host(d["W1"][ex]), _host(d["W2"][ex]),
                                        hh, pp, cfg.dtype)
        del x_rows, d_rows
        g1 = layer.grad1[ex] - init1[ex]
        got1 = np.stack([_host(g1[hh_d][:, torch.from_numpy(gate[pp]).cuda()]),
                         _host(g1[hh_d][:, torch.from_numpy(up[pp]).cuda()])], axis=1)
        got2 = _host((layer.grad2[ex] - init2[ex])[pp_d])
        e1 = float(np.abs(got1 - dW1).max() / max(np.sqrt(np.mean(dW1 ** 2)), 1e-30))
        e2 = float(np.abs(got2 - dW2).max() / max(np.sqrt(np.mean(dW2 ** 2)), 1e-30))
        say("ffn backward dW expert", ex, "slots", len(tok), "dW1", e1, "dW2", e2)
        assert max(e1, e2) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ffn_backward_small_full_compare(dtype):
    cfg = small_cfg(name=f"ffn_bwd_{dtype}", R=4, S=37, E=16, K=4, H=128, Hp=192, dtype=dtype)
    _ffn_backward_check(cfg, 3.0, alpha=2.5, full=True)


def test_ffn_backward_full_size_sampled():
    _ffn_backward_check(CONFIGS["train_backward"], 15.0)


@pytest.mark.parametrize("key", [("bench_shape", 20.0), ("infer_overflow", 10.0)],
                         ids=lambda k: f"{k[0]}-{k[1]}")
def test_ffn_forward_full_size_sampled(key):
    name, target = key
    cfg = CONFIGS[name]
    say("ffn forward sampled", name, target)
    r, layer, d, topk, gates = _setup(cfg, target)
    _poison(layer)
    y = layer.forward(topk, d["x"], gates)
    torch.cuda.synchronize()
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert np.array_equal(layer.slot_map.cpu().numpy(), pl.slot_map)
    if cfg.mode == "infer":
        assert pl.n_overflow >= 1
    rng = np.random.default_rng(1)
    N, K = cfg.R * cfg.S, cfg.K
    pick = set(rng.choice(N, 8, replace=False).tolist())
    for e in sorted(set(int(x) for x in pl.replica_expert.ravel() if x >= 0))[:2]:
        pick.add(int(np.nonzero((r.topk_idx == e).any(axis=1))[0][-1]))
    for e in range(cfg.E):     # overflow pieces: rows e < E on a non-home rank
        for (q, row, tlo, thi) in pl.pieces[e]:
            if row < cfg.E and q != e // cfg.G:
                pick.add(int(np.nonzero((r.topk_idx == e).any(axis=1))[0][tlo]))
                break
    toks = np.array(sorted(pick))
    slots = (toks[:, None] * K + np.arange(K)[None, :]).ravel()
    ref = _slot_oracle(d, cfg, r.topk_idx, slots)
    pos = torch.from_numpy(pl.slot_map[slots]).long().cuda()
    act_got, z_got = _host(layer.act[pos]), _host(layer.z[pos])
    act_ref = np.stack([ref[int(u)][1] for u in slots])
    z_ref = np.stack([ref[int(u)][2] for u in slots])
    assert_stored_close(act_got, act_ref, cfg.dtype, "act")
    assert rel_err(z_got, z_ref) <= tolerance(cfg)
    y_ref = np.stack([sum(float(r.gates[g, k]) * z_ref[i * K + k] for k in range(K))
                      for i, g in enumerate(toks)])
    err = rel_err(_host(y[torch.from_numpy(toks).cuda()]), y_ref)
    say("ffn forward sampled", name, target, len(toks), "tokens, max err / RMS", err)
    assert err <= tolerance(cfg)


def test_ffn_graph_capture_replays_match_eager():
    """The FFN's forward + backward captured in one HIP graph; three replays, each
    after eager work and a reset of the += gradient targets, equal the eager run
    bit for bit."""
    cfg = small_cfg(name="ffn_graph", R=4, S=96, E=16, K=4, H=128, Hp=192)
    say("ffn graph capture", cfg.name)
    r, layer, d, topk, gates = _setup(cfg, 3.0, backward=True, alpha=2.5)

    def run():
        layer.forward(topk, d["x"], gates)
        layer.backward(d["dyH"], gates)

    def reset():
        layer.grad1.zero_()
        layer.grad2.zero_()

    reset()
    run()
    torch.cuda.synchronize()
    keys = ("y", "dx", "grad1", "grad2", "act", "hs", "slot_map")
    want = {k: getattr(layer, k).clone() for k in keys}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset()
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        reset()
        layer.y.fill_(float("nan"))
        layer.dx.fill_(float("nan"))
        layer.act.fill_(0)
        _ = (torch.randn(4096, device="cuda") @ torch.randn(4096, 64, device="cuda")).sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in want.items():
            assert torch.equal(getattr(layer, k), v), (rep, k)
        assert int(torch.count_nonzero(layer.red1)) == 0
        assert int(torch.count_nonzero(layer.red2)) == 0
