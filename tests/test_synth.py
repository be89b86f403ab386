"""The seeded input generator: reproducible, hits its imbalance targets, and the
overflow profile really forces inference-mode overflow."""
import numpy as np
import pytest

from oracle import plan as P
from redundant_expert_balancing_amd.synth import CONFIGS, ALPHA, make_routing


def _tolerance(cfg, target):
    tbar = cfg.N * cfg.K / cfg.E
    return max(1.0 / tbar, 0.002 * (1.0 + target))


@pytest.mark.parametrize("key", sorted(ALPHA), ids=lambda k: f"{k[0]}-{k[1]}")
def test_routing_hits_target_imbalance(key):
    name, target = key
    cfg = CONFIGS[name]
    r = make_routing(cfg, target)
    assert r.topk_idx.shape == (cfg.N, cfg.K) and r.topk_idx.dtype == np.int32
    # distinct experts per token, ids in range
    srt = np.sort(r.topk_idx, axis=1)
    assert (np.diff(srt, axis=1) > 0).all() and srt.min() >= 0 and srt.max() < cfg.E
    # gates: softmax of the selected scores, descending in k, summing to 1
    assert np.allclose(r.gates.sum(axis=1), 1.0, atol=1e-6)
    assert (np.diff(r.gates, axis=1) <= 0).all()
    mv = P.maxvio(P.expert_loads(r.topk_idx, cfg.E), cfg.R, cfg.S, cfg.K, cfg.E)
    assert abs(mv - target) <= _tolerance(cfg, target), mv
    assert mv == pytest.approx(r.maxvio)


def test_routing_is_reproducible():
    cfg = CONFIGS["bf16_train_mild"]
    a = make_routing(cfg, 0.2)
    b = make_routing(cfg, 0.2)
    assert np.array_equal(a.topk_idx, b.topk_idx) and np.array_equal(a.gates, b.gates)
    c = make_routing(cfg, 0.2, seed=1)
    assert not np.array_equal(a.topk_idx, c.topk_idx)


def test_overflow_profile_forces_overflow():
    cfg = CONFIGS["infer_overflow"]
    r = make_routing(cfg, 10.0)
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    assert pl.n_overflow >= 1
