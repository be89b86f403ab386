"""GPU tests of the process-global prefetch-slot pool (virtual-memory views) and
of a layer stack whose prefetch runs on a side stream.

* views of one pool set alias the same slot memory while their home rows stay
  apart; views of different sets do not alias; the pool holds R*B rows per set
  whatever the number of layers;
* a stack of layers sharing the pool, forward then backward (which prefetches a
  layer's replicas again where a later layer overwrote them), gives bit for bit
  the outputs, input gradients and weight gradients of independent layers with
  private slots: one set with the prefetch serial or on a side stream, and two
  sets with the next layer's backward prefetch under the current layer's GEMMs;
  and every layer's y, dX and weight gradient equals the float64 oracle's dense
  values within the bf16 bar (max abs error <= 1e-2 * RMS(reference))
  [ai-maestro.online "Moonshot AI open-sources MoonEP", section "The memory
  contract": prefetch slots come from one process-global pool shared by all
  layers, and replicas change no result].
"""
import numpy as np
import pytest
import torch

from oracle import moe as M
from redundant_expert_balancing_amd import _lib as L
from redundant_expert_balancing_amd.layer import MoEProjection
from redundant_expert_balancing_amd.pool import MoEStack, PooledWeights, SlotPool
from redundant_expert_balancing_amd.synth import make_routing

from gpu_helpers import rel_err, say, small_cfg, tolerance

pytestmark = pytest.mark.gpu


def _pool_cfg(name, S=64, H=1024, Hp=1024, dtype="bf16"):
    """A layer whose home rows end on a mapping boundary (row = H*Hp elements)."""
    cfg = small_cfg(name=name, R=4, S=S, E=16, K=4, H=H, Hp=Hp, dtype=dtype)
    gran = L.moonep_vm_granularity()
    assert gran > 0, "device reports no virtual memory support"
    rb = H * Hp * (2 if dtype == "bf16" else 4)
    assert (cfg.E * rb) % gran == 0, (gran, rb)
    return cfg, gran, rb


def test_views_alias_slots_and_keep_homes_apart():
    cfg, gran, rb = _pool_cfg("pool_alias")
    say("pool alias", gran, rb)
    E, RB = cfg.E, cfg.R * cfg.B
    pool = SlotPool(cfg, 1)
    assert pool.nbytes == -(-RB * rb // gran) * gran
    a, b = PooledWeights(cfg, pool, 0), PooledWeights(cfg, pool, 0)
    try:
        assert a.tensor.shape == (E + RB, cfg.H, cfg.Hp)
        assert a.tensor.data_ptr() != b.tensor.data_ptr()
        a.tensor[:E].fill_(1.0)
        b.tensor[:E].fill_(2.0)
        g = torch.Generator(device="cuda").manual_seed(0)
        pat = torch.randn((RB, cfg.H, cfg.Hp), generator=g, device="cuda").to(torch.bfloat16)
        a.tensor[E:].copy_(pat)
        torch.cuda.synchronize()
        assert torch.equal(b.tensor[E:], pat)             # one slot memory
        assert bool((a.tensor[:E] == 1.0).all()) and bool((b.tensor[:E] == 2.0).all())
        b.tensor[E:].zero_()
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(a.tensor[E:])) == 0
    finally:
        a.close()
        b.close()
        pool.close()


def test_pool_sets_are_disjoint():
    cfg, gran, rb = _pool_cfg("pool_sets")
    say("pool sets")
    E = cfg.E
    pool = SlotPool(cfg, 2)
    a, b = PooledWeights(cfg, pool, 0), PooledWeights(cfg, pool, 1)
    try:
        assert pool.nbytes == 2 * (-(-cfg.R * cfg.B * rb // gran) * gran)
        a.tensor[E:].fill_(3.0)
        b.tensor[E:].fill_(4.0)
        torch.cuda.synchronize()
        assert bool((a.tensor[E:] == 3.0).all()) and bool((b.tensor[E:] == 4.0).all())
    finally:
        a.close()
        b.close()
        pool.close()


@pytest.mark.parametrize("overlap,nsets", [(True, 1), (False, 1), (True, 2)],
                         ids=["side_stream-1set", "serial-1set", "side_stream-2sets"])
def test_stack_matches_independent_layers(overlap, nsets):
    cfg, _, _ = _pool_cfg("pool_stack", S=96)
    n_layers = 4
    say("pool stack", "overlap" if overlap else "serial", nsets)
    kw = dict(overlap_forward=overlap, overlap_backward=overlap)
    E, W = cfg.E, cfg.E + cfg.R * cfg.B
    g = torch.Generator(device="cuda").manual_seed(11)
    ins = []
    for l in range(n_layers):
        r = make_routing(cfg, 3.0, seed=l, alpha=2.0 + 0.5 * l)
        w = (torch.randn((E, cfg.H, cfg.Hp), generator=g, device="cuda") * cfg.H ** -0.5).to(torch.bfloat16)
        x = torch.randn((cfg.N, cfg.H), generator=g, device="cuda").to(torch.bfloat16)
        dy = torch.randn((cfg.N, cfg.Hp), generator=g, device="cuda").to(torch.bfloat16)
        ins.append((torch.from_numpy(r.topk_idx).cuda(), torch.from_numpy(r.gates).cuda(), w, x, dy))
    stack = MoEStack(cfg, n_layers, backward=True, nsets=nsets, **kw)
    try:
        for l, (_, _, w, _, _) in enumerate(ins):
            stack.layers[l].w_all[:E].copy_(w)
            stack.layers[l].grad_home.zero_()
        for l, (topk, gates, _, x, _) in enumerate(ins):
            stack.forward_layer(l, topk, x, gates)
        for l in reversed(range(n_layers)):
            topk, gates, _, _, dy = ins[l]
            stack.backward_layer(l, dy, gates)
        torch.cuda.synchronize()
        for l, (topk, gates, w, x, dy) in enumerate(ins):
            w_all = torch.empty((W, cfg.H, cfg.Hp), dtype=torch.bfloat16, device="cuda")
            w_all[:E].copy_(w)
            ref = MoEProjection(cfg, "cuda", backward=True, w_all=w_all)
            ref.grad_home.zero_()
            ref.forward(topk, x, gates)
            ref.backward(dy, gates)
            torch.cuda.synchronize()
            s = stack.layers[l]
            assert int((ref.replica_expert[:, :cfg.B] >= 0).sum()) > 0
            for name in ("cu_seqlens", "slot_map", "replica_expert", "y", "dx", "grad_home"):
                assert torch.equal(getattr(s, name), getattr(ref, name)), (l, name)
            assert int(torch.count_nonzero(s.reduce_buf)) == 0
            del ref, w_all
            # the stacked layer against the oracle (inputs only: router output, x, W, dy)
            x_h, w_h, dy_h = (t.float().cpu().numpy() for t in (x, w, dy))
            topk_h, gates_h = topk.cpu().numpy(), gates.cpu().numpy()
            y_ref = M.dense_forward(x_h, w_h, topk_h, gates_h)
            dd = M.gated_dy(dy_h, gates_h, cfg.dtype)
            dx_ref, dW_ref = M.dense_backward(x_h, w_h, topk_h, dd)
            errs = [rel_err(s.y.cpu().numpy(), y_ref), rel_err(s.dx.cpu().numpy(), dx_ref),
                    rel_err(s.grad_home.cpu().numpy(), dW_ref)]
            say("pool stack layer", l, "vs oracle: y, dx, dW", errs)
            assert max(errs) <= tolerance(cfg)
    finally:
        stack.close()
