"""GPU value parity of the whole path: plan -> prefetch_weight -> dispatch ->
grouped GEMM -> combine, and the backward (gated dispatch of dY, dgrad, wgrad,
unpermute, reduce_grad), against the float64 oracle on the same inputs.

Small layers are compared element by element everywhere; the full-size layers on
sampled tokens and experts (the oracle computes those one by one), plus
properties that hold at any size (the permuted buffers are exact copies, the
prefetch slots equal their home rows, home rows are never written, consumed
replica-gradient slots end at zero). Tolerances: max abs error <= 1e-2 *
RMS(reference) for bf16 layers, <= 1e-5 * RMS(reference) for fp32 layers.
"""
import numpy as np
import pytest
import torch

from oracle import moe as M
from oracle import plan as P
from redundant_expert_balancing_amd import _lib as L
from redundant_expert_balancing_amd.layer import MoEProjection
from redundant_expert_balancing_amd.synth import CONFIGS, make_dense, make_routing

from gpu_helpers import LazyW, assert_plan_equal, rel_err, say, small_cfg, tolerance

pytestmark = pytest.mark.gpu


def _setup(cfg, target, backward=False, alpha=None, seed=0):
    r = make_routing(cfg, target, seed=seed, alpha=alpha)
    d = make_dense(cfg, "cuda", seed, which=("x", "W", "dy") if backward else ("x", "W"),
                   w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEProjection(cfg, "cuda", backward=backward, w_all=d["W"])
    topk = torch.from_numpy(r.topk_idx).cuda()
    gates = torch.from_numpy(r.gates).cuda()
    return r, layer, d, topk, gates


def _host(t):
    return t.float().cpu().numpy()


def _poison_forward(layer):
    layer.xp.view(torch.int16).fill_(-1)      # bf16 / fp32 NaN patterns
    layer.out.fill_(float("nan"))
    layer.y.fill_(float("nan"))


def _check_permuted_copy(layer, x, slot_map, K):
    """xp[slot_map[u]] == x[u // K] bit for bit, for every slot."""
    sm = slot_map.long()
    src = torch.arange(sm.numel(), device=sm.device) // K
    assert torch.equal(layer.xp[sm], x[src])


@pytest.mark.parametrize("name", ["tiny_fp32_train", "bf16_train_mild"])
def test_forward_full_compare(name):
    cfg = CONFIGS[name]
    target = cfg.maxvio[0]
    say("forward full", name)
    r, layer, d, topk, gates = _setup(cfg, target)
    _poison_forward(layer)
    w_home = d["W"][:cfg.E].clone()
    y = layer.forward(topk, d["x"], gates)
    torch.cuda.synchronize()
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert_plan_equal({"cu_seqlens": layer.cu_seqlens.cpu().numpy(),
                       "replica_expert": layer.replica_expert[:, :cfg.B].cpu().numpy(),
                       "slot_map": layer.slot_map.cpu().numpy(),
                       "src_index": layer.src_index.cpu().numpy()}, pl)
    assert torch.equal(d["W"][:cfg.E], w_home)
    x_h, W_h = _host(d["x"]), _host(w_home)
    # prefetch slots hold exact copies of their experts
    for q in range(cfg.R):
        for j in range(cfg.B):
            e = int(pl.replica_expert[q, j])
            if e >= 0:
                assert torch.equal(layer.w_all[cfg.E + q * cfg.B + j], w_home[e])
    _check_permuted_copy(layer, d["x"], layer.slot_map, cfg.K)
    # GEMM output of every slot, and the combined output, against the oracle
    out_ref = M.dense_expert_outputs(x_h, W_h, r.topk_idx)            # [N*K, H'] by slot u
    out_got = _host(layer.out)[pl.slot_map]
    assert rel_err(out_got, out_ref) <= tolerance(cfg)
    y_ref = M.dense_forward(x_h, W_h, r.topk_idx, r.gates)
    e = rel_err(_host(y), y_ref)
    say("forward full", name, "max err / RMS", e)
    assert e <= tolerance(cfg)


@pytest.mark.parametrize("key", [("bench_shape", 0.2), ("bench_shape", 1.0), ("bench_shape", 10.0),
                                 ("bench_shape", 20.0), ("infer_overflow", 10.0)],
                         ids=lambda k: f"{k[0]}-{k[1]}")
def test_forward_full_size_sampled(key):
    name, target = key
    cfg = CONFIGS[name]
    say("forward sampled", name, target)
    r, layer, d, topk, gates = _setup(cfg, target)
    w_home = d["W"][:cfg.E].clone()
    _poison_forward(layer)
    y = layer.forward(topk, d["x"], gates)
    torch.cuda.synchronize()
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert np.array_equal(layer.slot_map.cpu().numpy(), pl.slot_map)
    assert np.array_equal(layer.cu_seqlens.cpu().numpy(), pl.cu_seqlens)
    if cfg.mode == "infer":
        assert pl.n_overflow >= 1
    assert torch.equal(d["W"][:cfg.E], w_home)
    for q in range(cfg.R):
        for j in range(cfg.B):
            e = int(pl.replica_expert[q, j])
            if e >= 0:
                assert torch.equal(layer.w_all[cfg.E + q * cfg.B + j], w_home[e])
    _check_permuted_copy(layer, d["x"], layer.slot_map, cfg.K)
    # sampled tokens: spread over all ranks, plus tokens routed to replicated and
    # overflow experts (their slots land in prefetch rows or remote home rows)
    rng = np.random.default_rng(1)
    N = cfg.R * cfg.S
    pick = set(rng.choice(N, 12, replace=False).tolist())
    rep_experts = set(int(e) for e in pl.replica_expert.ravel() if e >= 0)
    for e in sorted(rep_experts)[:4]:
        pick.add(int(np.nonzero((r.topk_idx == e).any(axis=1))[0][-1]))
    for e in range(cfg.E):     # overflow pieces: rows e < E on a non-home rank
        for (q, row, tlo, thi) in pl.pieces[e]:
            if row < cfg.E and q != e // cfg.G:
                toks = np.nonzero((r.topk_idx == e).any(axis=1))[0]
                pick.add(int(toks[tlo]))
    toks = np.array(sorted(pick))
    W = LazyW(w_home)
    x_s = _host(d["x"][torch.from_numpy(toks).cuda()])
    out_ref = M.dense_expert_outputs(x_s, W, r.topk_idx[toks])
    slots = (toks[:, None] * cfg.K + np.arange(cfg.K)[None, :]).ravel()
    out_got = _host(layer.out[torch.from_numpy(pl.slot_map[slots]).long().cuda()])
    assert rel_err(out_got, out_ref) <= tolerance(cfg)
    y_ref = M.dense_forward(x_s, W, r.topk_idx[toks], r.gates[toks])
    e = rel_err(_host(y[torch.from_numpy(toks).cuda()]), y_ref)
    say("forward sampled", name, target, len(toks), "tokens, max err / RMS", e)
    assert e <= tolerance(cfg)


def _backward_check(cfg, target, alpha=None, full=False):
    say("backward", cfg.name, target, "full" if full else "sampled")
    r, layer, d, topk, gates = _setup(cfg, target, backward=True, alpha=alpha)
    g0 = torch.Generator(device="cuda").manual_seed(123)
    init = torch.randn(layer.grad_home.shape, generator=g0, device="cuda")
    layer.grad_home.copy_(init)            # grads accumulate (+=) into whatever is there
    layer.forward(topk, d["x"], gates)
    layer.dyp.view(torch.int16).fill_(-1)
    layer.dxp.fill_(float("nan"))
    layer.dx.fill_(float("nan"))
    dx = layer.backward(d["dy"], gates)
    torch.cuda.synchronize()
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert pl.n_replicas > 0
    # consumed replica-gradient slots end at exactly zero
    assert int(torch.count_nonzero(layer.reduce_buf)) == 0
    # gated permute of dY: one fp32 product, one rounding; exact at every slot
    sm = layer.slot_map.long()
    u = torch.arange(sm.numel(), device="cuda")
    want = (gates.reshape(-1)[u][:, None] * d["dy"].float()[u // cfg.K]).to(layer.dtype)
    assert torch.equal(layer.dyp[sm], want)
    N = cfg.R * cfg.S
    rng = np.random.default_rng(2)
    toks = np.arange(N) if full else np.sort(rng.choice(N, 16, replace=False))
    tk = torch.from_numpy(toks).cuda()
    W = LazyW(d["W"][:cfg.E])
    x_s, dy_s = _host(d["x"][tk]), _host(d["dy"][tk])
    dd = M.gated_dy(dy_s, r.gates[toks], cfg.dtype)
    # dgrad oracle: dx[g] = sum_k d(g,k) @ W[e]^T
    if full:
        dx_ref, _ = M.dense_backward(x_s, np.stack([W[e] for e in range(cfg.E)]),
                                     r.topk_idx[toks], dd)
    else:
        dx_ref = np.zeros((len(toks), cfg.H))
        for i, g in enumerate(toks):
            for k in range(cfg.K):
                w_e = W[r.topk_idx[g, k]].astype(np.float64)
                dx_ref[i] += dd[i * cfg.K + k].astype(np.float64) @ w_e.T
    e = rel_err(_host(dx[tk]), dx_ref)
    say("backward dx err", e)
    assert e <= tolerance(cfg)
    # weight gradients: replicated experts (gradient folded home) and a few others
    experts = sorted(set(int(x) for x in pl.replica_expert.ravel() if x >= 0))[:6]
    experts += [int(x) for x in rng.choice(cfg.E, 3, replace=False) if x not in experts]
    hh = rng.choice(cfg.H, 24, replace=False)
    pp = rng.choice(cfg.Hp, 24, replace=False)
    gh = layer.grad_home
    for ex in experts:
        tok, kk = np.nonzero(r.topk_idx == ex)
        if len(tok) == 0:
            continue
        t_dev = torch.from_numpy(tok).cuda()
        x_rows = _host(d["x"][t_dev][:, torch.from_numpy(hh).cuda()])
        dy_rows = _host(d["dy"][t_dev][:, torch.from_numpy(pp).cuda()])
        d_all = M.gated_dy(dy_rows, r.gates[tok], cfg.dtype)          # [n*K, |pp|]
        d_rows = d_all[np.arange(len(tok)) * cfg.K + kk]
        ref = _host(init[ex][torch.from_numpy(hh).cuda()][:, torch.from_numpy(pp).cuda()]) + \
            M.wgrad_entries(x_rows, d_rows, np.arange(len(hh)), np.arange(len(pp)))
        got = _host(gh[ex][torch.from_numpy(hh).cuda()][:, torch.from_numpy(pp).cuda()])
        scale = M.wgrad_entries(x_rows, d_rows, np.arange(len(hh)), np.arange(len(pp)))
        err = float(np.abs(got - ref).max() / max(np.sqrt(np.mean(scale ** 2)), 1e-30))
        say("backward dW expert", ex, "slots", len(tok), "err", err)
        assert err <= tolerance(cfg)


def test_backward_full_size_sampled():
    _backward_check(CONFIGS["train_backward"], 15.0)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_small_full_compare(dtype):
    cfg = small_cfg(name=f"bwd_small_{dtype}", R=4, S=96, E=16, K=4, H=128, Hp=192, dtype=dtype)
    _backward_check(cfg, 3.0, alpha=2.5, full=True)


def test_whole_layer_graph_capture_replays_match_eager():
    """Forward + backward captured in one HIP graph; three replays, each after
    eager work and a reset of the += gradient targets, equal the eager run bit
    for bit (the path is deterministic and never synchronises with the host)."""
    cfg = small_cfg(name="graph", R=4, S=96, E=16, K=4, H=128, Hp=192)
    say("graph capture", cfg.name)
    r, layer, d, topk, gates = _setup(cfg, 3.0, backward=True, alpha=2.5)

    def run():
        layer.forward(topk, d["x"], gates)
        layer.backward(d["dy"], gates)

    layer.grad_home.zero_()
    run()
    torch.cuda.synchronize()
    want = {k: getattr(layer, k).clone() for k in ("y", "dx", "grad_home", "cu_seqlens", "slot_map")}
    assert int(torch.count_nonzero(layer.reduce_buf)) == 0
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.grad_home.zero_()
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        layer.grad_home.zero_()
        layer.y.fill_(float("nan"))
        layer.dx.fill_(float("nan"))
        layer.slot_map.fill_(-5)
        _ = (torch.randn(4096, device="cuda") @ torch.randn(4096, 64, device="cuda")).sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in want.items():
            assert torch.equal(getattr(layer, k), v), (rep, k)
        assert int(torch.count_nonzero(layer.reduce_buf)) == 0


def test_per_rank_subproblems_reproduce_the_full_gemm():
    """The per-rank views used by the no-redundancy baseline: each balanced rank's
    one-rank GEMM equals its rows of the full grouped GEMM; each home-only rank's
    GEMM equals its rows of the one-rank (counting-sort) plan's GEMM; and that plan
    computes every (token, k) slot to the same bits as the balanced plan. Against
    the oracle: the plain-EP rank loads are oracle.plan.home_only_loads, and every
    row of every per-rank problem, balanced and plain EP, is x[g] @ W[e] of the slot
    the oracle's plan puts there [ai-maestro.online "Moonshot AI open-sources
    MoonEP", section "The problem MoonEP targets": with plain EP the hottest rank
    holds all of its experts' tokens]."""
    from redundant_expert_balancing_amd.baseline import balanced_rank, home_only_ranks
    from redundant_expert_balancing_amd.synth import LayerConfig
    cfg = CONFIGS["bf16_train_mild"]
    say("per-rank subproblems", cfg.name)
    r, layer, d, topk, gates = _setup(cfg, 0.2)
    layer.forward(topk, d["x"], gates)
    one = LayerConfig("one_rank", 1, cfg.N, cfg.E, cfg.K, 0, cfg.H, cfg.Hp, cfg.dtype, "infer", (0.2,))
    layer1 = MoEProjection(one, "cuda", w_all=d["W"][:cfg.E])
    layer1.forward(topk, d["x"], gates)
    torch.cuda.synchronize()
    SK = cfg.S * cfg.K
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    pl1 = P.plan(r.topk_idx, 1, cfg.N, cfg.E, cfg.K, 0, "infer")
    assert np.array_equal(layer.src_index.cpu().numpy(), pl.src_index)
    assert np.array_equal(layer1.src_index.cpu().numpy(), pl1.src_index)
    # every slot's oracle value, indexed by flat slot id u = g*K + k
    out_ref = M.dense_expert_outputs(_host(d["x"]), _host(d["W"][:cfg.E]), r.topk_idx)
    for q in range(cfg.R):
        p = balanced_rank(layer, q)
        p.run()
        torch.cuda.synchronize()
        assert torch.equal(p.out, layer.out[q * SK:(q + 1) * SK]), q
        e = rel_err(_host(p.out), out_ref[pl.src_index[q * SK:(q + 1) * SK]])
        assert e <= tolerance(cfg), ("balanced rank", q, e)
    probs, rows = home_only_ranks(cfg, layer1.xp, layer1.cu_seqlens[0], d["W"])
    assert rows == P.home_only_loads(r.topk_idx, cfg.R, cfg.E)
    assert sum(rows) == cfg.N * cfg.K
    start = 0
    for q, p in enumerate(probs):
        p.run()
        torch.cuda.synchronize()
        assert torch.equal(p.out[:rows[q]], layer1.out[start:start + rows[q]]), q
        e = rel_err(_host(p.out[:rows[q]]), out_ref[pl1.src_index[start:start + rows[q]]])
        say("plain-EP rank", q, "rows", rows[q], "max err / RMS", e)
        assert e <= tolerance(cfg), ("plain-EP rank", q, e)
        start += rows[q]
    assert torch.equal(layer1.out[layer1.slot_map.long()], layer.out[layer.slot_map.long()])
    assert rows == pl.L


@pytest.mark.parametrize("kw", [
    dict(R=4, S=40, E=1024, K=8, H=64, Hp=64),                 # largest expert count, B = 256
    dict(R=2, S=53, E=8, K=1, H=320, Hp=192),                  # K = 1; H, H' end inside a tile
    dict(R=2, S=24, E=64, K=32, H=64, Hp=128),                 # K = 32
    dict(R=1, S=77, E=16, K=4, B=0, H=128, Hp=64, mode="infer"),   # one rank, no slots
    dict(R=8, S=33, E=32, K=2, B=1, H=192, Hp=320, mode="infer"),  # overflow into home rows
    dict(R=8, S=30, E=928, K=8, B=95, H=64, Hp=64, mode="infer"),  # R*(E+B+1) = 8192, the limit
    dict(R=64, S=8, E=64, K=2, H=64, Hp=128),                  # 64 ranks of one expert, B = 1
    dict(R=8, S=16384, E=64, K=8, H=64, Hp=64),                # over 4096 tile-list entries:
                                                               # the list built in memory
], ids=["E1024", "K1_ragged_tiles", "K32", "R1_B0", "infer_B1", "rows_limit", "R64",
        "tile_list_in_memory"])
def test_edge_shapes_full_compare(kw):
    """Forward (and backward where the layer trains) compared element by element with
    the oracle at edge shapes of the plan and of the GEMM tiling."""
    cfg = small_cfg(name="edge", **kw)
    say("edge shape", kw)
    alpha = 2.0 if cfg.E <= 64 else 4.0
    bwd = cfg.mode == "train"
    r, layer, d, topk, gates = _setup(cfg, 3.0, backward=bwd, alpha=alpha)
    if bwd:
        layer.grad_home.zero_()
    _poison_forward(layer)
    y = layer.forward(topk, d["x"], gates)
    if bwd:
        dx = layer.backward(d["dy"], gates)
    torch.cuda.synchronize()
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert np.array_equal(layer.slot_map.cpu().numpy(), pl.slot_map)
    assert np.array_equal(layer.cu_seqlens.cpu().numpy(), pl.cu_seqlens)
    x_h, W_h = _host(d["x"]), _host(d["W"][:cfg.E])
    y_ref = M.dense_forward(x_h, W_h, r.topk_idx, r.gates)
    assert rel_err(_host(y), y_ref) <= tolerance(cfg)
    if bwd:
        dd = M.gated_dy(_host(d["dy"]), r.gates, cfg.dtype)
        dx_ref, dW_ref = M.dense_backward(x_h, W_h, r.topk_idx, dd)
        assert rel_err(_host(dx), dx_ref) <= tolerance(cfg)
        assert rel_err(_host(layer.grad_home), dW_ref) <= tolerance(cfg)
        assert int(torch.count_nonzero(layer.reduce_buf)) == 0


def _random_layer_kwargs(i):
    """Seeded random small layer: R in 1..8, G = E/R in 1..16, K <= min(E, 8), S in
    1..160, H and H' multiples of 64 up to 448 (partial 256-column tiles, odd numbers of
    64-deep k-steps), training (B = G) or inference (B in 0..G); mostly bfloat16."""
    rng = np.random.default_rng(1000 + i)
    R = int(rng.choice([1, 2, 3, 4, 8]))
    G = int(rng.integers(1, 17))
    E = R * G
    K = int(rng.integers(1, min(E, 8) + 1))
    train = bool(rng.random() < 0.7)
    B = G if train else int(rng.integers(0, G + 1))
    return dict(R=R, S=int(rng.integers(1, 161)), E=E, K=K, B=B,
                H=64 * int(rng.integers(1, 8)), Hp=64 * int(rng.integers(1, 8)),
                dtype="fp32" if rng.random() < 0.15 else "bf16",
                mode="train" if train else "infer")


@pytest.mark.parametrize("i", range(24))
def test_random_layers_full_compare(i):
    """Forward (and backward where the layer trains) of seeded random small layers,
    every output element compared with the oracle: plan bit-exact, y, dx and the
    weight gradients within the layer's tolerance, replica-gradient slots zero."""
    from redundant_expert_balancing_amd import _lib as L
    kw = _random_layer_kwargs(i)
    cfg = small_cfg(name=f"random{i}", **kw)
    assert L.moonep_validate_shape(L.Shape.of(cfg)) == L.OK
    say("random layer", i, kw)
    bwd = cfg.mode == "train"
    r, layer, d, topk, gates = _setup(cfg, 3.0, backward=bwd, alpha=float(1 + i % 4), seed=i)
    if bwd:
        layer.grad_home.zero_()
    _poison_forward(layer)
    y = layer.forward(topk, d["x"], gates)
    if bwd:
        dx = layer.backward(d["dy"], gates)
    torch.cuda.synchronize()
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert np.array_equal(layer.slot_map.cpu().numpy(), pl.slot_map)
    assert np.array_equal(layer.cu_seqlens.cpu().numpy(), pl.cu_seqlens)
    x_h, W_h = _host(d["x"]), _host(d["W"][:cfg.E])
    y_ref = M.dense_forward(x_h, W_h, r.topk_idx, r.gates)
    assert rel_err(_host(y), y_ref) <= tolerance(cfg)
    if bwd:
        dd = M.gated_dy(_host(d["dy"]), r.gates, cfg.dtype)
        dx_ref, dW_ref = M.dense_backward(x_h, W_h, r.topk_idx, dd)
        assert rel_err(_host(dx), dx_ref) <= tolerance(cfg)
        # experts no token chose keep their gradient exactly (zero), and the whole
        # gradient is within the layer's bar
        gh = _host(layer.grad_home)
        idle = np.setdiff1d(np.arange(cfg.E), np.unique(r.topk_idx))
        assert not np.any(gh[idle])
        assert rel_err(gh, dW_ref) <= tolerance(cfg)
        assert int(torch.count_nonzero(layer.reduce_buf)) == 0


def test_binding_refuses_wrong_buffers():
    """Buffers too small, of the wrong dtype or not contiguous are refused by the
    binding before any launch; the layer still works afterwards."""
    cfg = CONFIGS["bf16_train_mild"]
    say("binding checks")
    r, layer, d, topk, gates = _setup(cfg, cfg.maxvio[0])
    sh = layer.shape
    x = d["x"]
    with pytest.raises(ValueError, match="bytes"):
        L.moonep_dispatch(sh, cfg.H, x, layer.slot_map, None, layer.xp[: layer.xp.shape[0] // 2])
    with pytest.raises(ValueError, match="dtype"):
        L.moonep_dispatch(sh, cfg.H, x.float(), layer.slot_map, None, layer.xp)
    with pytest.raises(ValueError, match="contiguous"):
        L.moonep_combine(sh, cfg.Hp, layer.out.t(), layer.slot_map, gates, layer.y)
    with pytest.raises(ValueError, match="bytes"):
        L.moonep_grouped_gemm(sh, L.FWD, layer.xp, layer.w_all[: cfg.E], layer.cu_seqlens,
                              layer.out, None, None, layer.ws)
    with pytest.raises(ValueError, match="bytes"):
        L.moonep_plan(sh, topk, layer.cu_seqlens, layer.replica_expert, layer.slot_map,
                      layer.src_index, layer.ws[:16])
    y = layer.forward(topk, x, gates)
    torch.cuda.synchronize()
    assert layer.error_flags() == 0
    x_h, W_h = _host(x), _host(d["W"][:cfg.E])
    assert rel_err(_host(y), M.dense_forward(x_h, W_h, r.topk_idx, r.gates)) <= tolerance(cfg)
