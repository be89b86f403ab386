"""moonep_grouped_gemm_noalloc (tile lists in the library's static per-device scratch
array, no workspace, nothing allocated) against moonep_grouped_gemm (tile lists in the
caller's workspace) through the C ABI: the same kernels, so every output must be bit
for bit equal. Two calls in a row share the scratch array, the second with a smaller
layer, so lists left over from the first call must not leak into the second.
"""
import pytest
import torch

from redundant_expert_balancing_amd import _lib as L
from redundant_expert_balancing_amd.layer import MoEProjection
from redundant_expert_balancing_amd.synth import make_dense, make_routing

from gpu_helpers import say, small_cfg

pytestmark = pytest.mark.gpu


def _planned_layer(cfg, alpha, seed=0):
    r = make_routing(cfg, 3.0, seed=seed, alpha=alpha)
    d = make_dense(cfg, "cuda", seed, which=("x", "W", "dy"), w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEProjection(cfg, "cuda", backward=cfg.mode == "train", w_all=d["W"])
    topk, gates = torch.from_numpy(r.topk_idx).cuda(), torch.from_numpy(r.gates).cuda()
    layer.plan(topk)
    layer.prefetch()
    layer.dispatch(d["x"])
    if cfg.mode == "train":
        L.moonep_dispatch(layer.shape, cfg.Hp, d["dy"], layer.slot_map, gates, layer.dyp)
    return layer


def _both(layer, op):
    """(workspace result, scratch result) of one grouped GEMM op, outputs poisoned first."""
    c = layer.cfg
    res = []
    for noalloc in (False, True):
        if op == L.WGRAD:
            g = torch.Generator(device="cuda").manual_seed(9)
            gh = torch.randn(layer.grad_home.shape, generator=g, device="cuda")
            rb = torch.zeros_like(layer.reduce_buf)
            a, b, out = layer.xp, layer.dyp, None
        else:
            gh = rb = None
            a = layer.xp if op == L.FWD else layer.dyp
            b = layer.w_all
            out = torch.full((layer.xp.shape[0], c.Hp if op == L.FWD else c.H), float("nan"),
                             device="cuda")
        if noalloc:
            L.moonep_grouped_gemm_noalloc(layer.shape, op, a, b, layer.cu_seqlens, out, gh, rb)
        else:
            L.moonep_grouped_gemm(layer.shape, op, a, b, layer.cu_seqlens, out, gh, rb, layer.ws)
        torch.cuda.synchronize()
        res.append((out, gh, rb))
    return res


def _assert_same(res, what):
    (o0, g0, r0), (o1, g1, r1) = res
    for x, y, name in ((o0, o1, "out"), (g0, g1, "grad_home"), (r0, r1, "reduce_buf")):
        if x is not None:
            assert torch.equal(x, y), (what, name)
    if o0 is not None:
        assert bool(torch.isfinite(o1).all()), what


# first call: a layer whose GEMMs split short tails into their own list (bf16, four
# rounds of full tiles); second call: a smaller layer without the split; third: float32
CALLS = [
    dict(name="large_tails", R=8, S=3072, E=128, K=8, H=384, Hp=320, alpha=1.0),
    dict(name="smaller", R=4, S=200, E=16, K=4, H=128, Hp=192, alpha=2.5),
    dict(name="fp32_smaller", R=4, S=96, E=16, K=2, H=128, Hp=64, alpha=2.0, dtype="fp32"),
]


def test_noalloc_gemm_matches_workspace_gemm_on_consecutive_calls():
    for kw in CALLS:
        kw = dict(kw)
        name, alpha = kw.pop("name"), kw.pop("alpha")
        cfg = small_cfg(name=name, **kw)
        say("noalloc gemm", name, kw)
        layer = _planned_layer(cfg, alpha)
        for op in (L.FWD, L.DGRAD, L.WGRAD):
            say("noalloc gemm", name, "op", op)
            _assert_same(_both(layer, op), (name, op))
        del layer
        torch.cuda.empty_cache()


def test_noalloc_gemm_inference_overflow_and_empty_layer():
    """An inference layer with overflow rows (B = 1), then an empty layer (S = 0), which
    returns at once and leaves the output untouched."""
    cfg = small_cfg(name="infer_B1", R=8, S=33, E=32, K=2, B=1, H=192, Hp=320, mode="infer")
    say("noalloc gemm", cfg.name)
    layer = _planned_layer(cfg, 2.0)
    _assert_same(_both(layer, L.FWD), cfg.name)
    empty = small_cfg(name="empty", R=2, S=0, E=4, K=2, H=64, Hp=64)
    sh = L.Shape.of(empty)
    i32 = dict(dtype=torch.int32, device="cuda")
    cu = torch.zeros((empty.R, empty.E + empty.B + 1), **i32)
    xp = torch.zeros((1, empty.H), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((empty.E + empty.R * empty.B, empty.H, empty.Hp), dtype=torch.bfloat16,
                    device="cuda")
    out = torch.full((1, empty.Hp), 7.0, device="cuda")
    L.moonep_grouped_gemm_noalloc(sh, L.FWD, xp, w, cu, out, None, None)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
