"""GPU planner parity: moonep_plan bit-exact against the oracle plan.

Every layer configuration and imbalance point at full size, ragged and edge
shapes, invalid router data, determinism and HIP-graph capture. Outputs are
poison-filled before every call so unwritten entries are caught.
"""
import numpy as np
import pytest
import torch

from oracle import plan as P
from oracle.check import check_plan, check_order
from redundant_expert_balancing_amd import _lib as L
from redundant_expert_balancing_amd.layer import MoEProjection
from redundant_expert_balancing_amd.synth import ALPHA, CONFIGS, make_routing

from gpu_helpers import assert_plan_equal, plan_on_gpu, say, small_cfg

pytestmark = pytest.mark.gpu


class PlanOnly(MoEProjection):
    """Plan buffers only (no dense tensors)."""

    def __init__(self, cfg):
        self.cfg = cfg
        self.shape = L.Shape.of(cfg)
        self.device = torch.device("cuda")
        i32 = dict(dtype=torch.int32, device=self.device)
        N = cfg.R * cfg.S
        self.cu_seqlens = torch.empty((cfg.R, cfg.E + cfg.B + 1), **i32)
        self.replica_expert = torch.empty((cfg.R, max(cfg.B, 1)), **i32)
        self.slot_map = torch.empty((max(N * cfg.K, 1),), **i32)
        self.src_index = torch.empty((max(N * cfg.K, 1),), **i32)
        self.ws = torch.empty((L.moonep_workspace_bytes(self.shape) // 4,), **i32)
        L.moonep_workspace_init(self.shape, self.ws)


@pytest.mark.parametrize("key", sorted(ALPHA), ids=lambda k: f"{k[0]}-{k[1]}")
def test_plan_matches_oracle_full_size(key):
    name, target = key
    cfg = CONFIGS[name]
    say("plan", name, target)
    r = make_routing(cfg, target)
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    layer = PlanOnly(cfg)
    got, _ = plan_on_gpu(layer, r.topk_idx)
    assert_plan_equal(got, pl)
    assert layer.error_flags() == 0


def _random_topk(rng, N, E, K, hot=None):
    p = None
    if hot is not None:
        p = np.ones(E)
        p[hot] = 30.0
        p /= p.sum()
    return np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(N)]).astype(np.int32)


EDGE = [
    # (R, S, E, K, mode, B, hot experts)
    (4, 37, 16, 2, "train", None, [0, 1]),      # ragged: 148 tokens, not a multiple of 64
    (1, 100, 7, 3, "train", None, None),         # one rank: a stable counting sort
    (3, 1, 6, 2, "train", None, None),           # one token per rank
    (8, 64, 64, 1, "train", None, [5]),          # K = 1
    (2, 50, 64, 32, "train", None, None),        # K = 32 (largest)
    (4, 200, 1024, 8, "train", None, list(range(10))),  # E = 1024 (largest), 10-bit ids
    (16, 33, 256, 8, "infer", 0, list(range(16))),      # inference with no prefetch slot
    (16, 33, 256, 8, "infer", 4, list(range(16))),      # inference overflow
    (5, 129, 25, 4, "infer", 2, [0, 1, 2, 3, 4]),       # odd sizes everywhere
    (32, 8, 128, 4, "train", None, [0]),         # many ranks
    (64, 16, 64, 2, "train", None, [0, 1]),      # 64 ranks of one expert each (B = 1)
    (8, 100, 928, 8, "infer", 95, list(range(40))),  # R*(E+B+1) = 8192, the size limit
    # layers of at most 256 chunks of 64 tokens count, scan and solve in one launch of
    # 16-chunk workgroups; larger ones, or ones whose 16 histograms overflow 60 KiB of
    # LDS, take four launches
    (8, 296, 128, 6, "infer", 3, [0, 1, 2]),     # 37 chunks: a last workgroup of 5
    (8, 2048, 64, 4, "train", None, [0, 1, 2]),  # 256 chunks: the largest one-launch plan
    (1, 16385, 8, 2, "train", None, [0]),        # 257 chunks: four launches
    (8, 40, 960, 8, "infer", 0, list(range(20))),  # histograms fill the 60 KiB exactly
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"R{c[0]}S{c[1]}E{c[2]}K{c[3]}{c[4]}B{c[5]}")
def test_plan_edge_shapes(case):
    R, S, E, K, mode, B, hot = case
    cfg = small_cfg(R=R, S=S, E=E, K=K, mode=mode, B=B)
    rng = np.random.default_rng(R * 1000 + S)
    topk = _random_topk(rng, R * S, E, K, hot)
    say("plan edge", case)
    pl = P.plan(topk, R, S, E, K, cfg.B, mode)
    got, _ = plan_on_gpu(PlanOnly(cfg), topk)
    assert_plan_equal(got, pl)
    assert check_plan(topk, R, S, E, K, cfg.B, mode, got["cu_seqlens"], got["replica_expert"],
                      got["slot_map"], got["src_index"]) == []
    assert check_order(got["cu_seqlens"], got["src_index"], R, S, K, E, cfg.B) == []


def test_plan_balanced_and_star():
    R, S, E, K = 4, 16, 8, 2
    G = E // R
    balanced = np.array([[((r + s) % R) * G, ((r + s) % R) * G + 1] for r in range(R)
                         for s in range(S)], dtype=np.int32)
    rng = np.random.default_rng(2)
    star = _random_topk(rng, R * S, G, K)     # everything routed to group 0
    for topk in (balanced, star):
        cfg = small_cfg(R=R, S=S, E=E, K=K)
        pl = P.plan(topk, R, S, E, K, G, "train")
        got, _ = plan_on_gpu(PlanOnly(cfg), topk)
        assert_plan_equal(got, pl)
    assert (got["replica_expert"] >= 0).sum() > 0


def test_plan_empty_layer():
    """S = 0 in both modes: the plan equals the oracle's (all rows empty, no slots)."""
    for mode, B in (("train", None), ("infer", 2)):
        cfg = small_cfg(R=4, S=0, E=16, K=2, B=B, mode=mode)
        layer = PlanOnly(cfg)
        topk = np.zeros((0, 2), dtype=np.int32)
        got, _ = plan_on_gpu(layer, topk)
        assert_plan_equal(got, P.plan(topk, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode))
        assert (got["cu_seqlens"] == 0).all()
        assert (got["replica_expert"] == -1).all()


def test_plan_invalid_ids_flagged_and_plan_emptied():
    cfg = small_cfg(R=4, S=40, E=16, K=2)
    rng = np.random.default_rng(0)
    topk = _random_topk(rng, cfg.R * cfg.S, cfg.E, cfg.K)
    layer = PlanOnly(cfg)
    bad = topk.copy()
    bad[17, 1] = cfg.E           # out of range
    got, _ = plan_on_gpu(layer, bad)
    assert layer.error_flags(clear=True) & L.ERR_ID_RANGE
    assert (got["cu_seqlens"] == 0).all() and (got["slot_map"] == -1).all()
    assert (got["src_index"] == -1).all() and (got["replica_expert"] == -1).all()
    assert layer.error_flags() == 0
    dup = topk.copy()
    dup[5, 1] = dup[5, 0]        # the same expert twice in one row
    got, _ = plan_on_gpu(layer, dup)
    assert layer.error_flags(clear=True) == L.ERR_ID_DUP
    # a repeated id does not break the slot bijection
    assert sorted(got["slot_map"].tolist()) == list(range(cfg.R * cfg.S * cfg.K))
    got, _ = plan_on_gpu(layer, topk)
    assert layer.error_flags() == 0
    assert_plan_equal(got, P.plan(topk, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode))


def test_plan_deterministic_and_graph_capturable():
    cfg = CONFIGS["bf16_train_mild"]
    r = make_routing(cfg, 0.2)
    layer = PlanOnly(cfg)
    a, topk = plan_on_gpu(layer, r.topk_idx)
    b, _ = plan_on_gpu(layer, r.topk_idx)
    for k in a:
        assert np.array_equal(a[k], b[k])
    # capture the plan in a graph; replay with eager work and syncs in between
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.plan(topk)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        layer.plan(topk)
    for rep in range(3):
        for t in (layer.cu_seqlens, layer.slot_map, layer.src_index, layer.replica_expert):
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(layer.slot_map.cpu().numpy(), a["slot_map"]), rep
        assert np.array_equal(layer.src_index.cpu().numpy(), a["src_index"]), rep
        assert np.array_equal(layer.cu_seqlens.cpu().numpy(), a["cu_seqlens"]), rep
        _ = torch.ones(1000, device="cuda").sum().item()   # eager work between replays


def _gumbel_topk(rng, N, E, K, logp):
    """K distinct experts per token, drawn without replacement with probabilities
    exp(logp) (Gumbel top-K)."""
    keys = logp[None, :] + rng.gumbel(size=(N, E))
    return np.argpartition(-keys, K - 1, axis=1)[:, :K].astype(np.int32)


def test_plan_matches_oracle_random_layers():
    """60 seeded random layers within the size limits: ranks 2..32, experts per rank 1..8, K 1..8, ragged S,
    training and every inference B, skews from balanced to a few very hot experts
    (random Dirichlet weights), so deficits chain across several hot ranks and
    donors run to exactly zero excess in some of them."""
    rng = np.random.default_rng(2024)
    layers = 0
    case = -1
    while layers < 60:
        case += 1
        R = int(rng.choice([2, 3, 4, 5, 8, 16, 32]))
        G = int(rng.choice([1, 2, 3, 4, 8]))
        E = R * G
        K = int(rng.integers(1, min(E, 8) + 1))
        S = int(rng.integers(1, 120))
        mode = "train" if rng.random() < 0.5 else "infer"
        B = G if mode == "train" else int(rng.integers(0, G + 1))
        conc = float(rng.choice([0.05, 0.3, 1.0, 10.0]))
        logp = np.log(rng.dirichlet(np.full(E, conc)) + 1e-12)
        topk = _gumbel_topk(rng, R * S, E, K, logp)
        cfg = small_cfg(name=f"rand{case}", R=R, S=S, E=E, K=K, B=B, H=64, Hp=64, mode=mode)
        if L.moonep_validate_shape(L.Shape.of(cfg)) != L.OK:   # beyond a documented limit
            continue
        say("random plan", case, dict(R=R, G=G, K=K, S=S, mode=mode, B=B, conc=conc))
        pl = P.plan(topk, R, S, E, K, B, mode)
        assert check_plan(topk, R, S, E, K, B, mode, pl.cu_seqlens, pl.replica_expert,
                          pl.slot_map, pl.src_index) == []
        layer = PlanOnly(cfg)
        got, _ = plan_on_gpu(layer, topk)
        assert_plan_equal(got, pl)
        assert layer.error_flags() == 0
        layers += 1
    assert layers == 60
