"""Shared pieces of the GPU parity tests (not a test module)."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from redundant_expert_balancing_amd import _lib as L
from redundant_expert_balancing_amd.layer import MoEProjection
from redundant_expert_balancing_amd.synth import CONFIGS, LayerConfig, make_routing, make_dense

POISON_I32 = 0x5A5A5A5A


def say(*a):
    """Name the case before each GPU step, flushed, so a crash still says where."""
    print("[gpu]", *a, flush=True)


def small_cfg(name="adhoc", R=4, S=37, E=16, K=2, B=None, H=64, Hp=64, dtype="bf16",
              mode="train"):
    G = E // R
    return LayerConfig(name, R, S, E, K, G if B is None else B, H, Hp, dtype, mode, (1.0,))


class LazyW:
    """W[e] fetched from a device tensor on demand (home rows are inputs)."""

    def __init__(self, w_dev):
        self.w = w_dev
        self.shape = tuple(w_dev.shape)
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = self.w[e].float().cpu().numpy()
        return self.cache[e]


def poison_plan(layer: MoEProjection):
    for t in (layer.cu_seqlens, layer.replica_expert, layer.slot_map, layer.src_index):
        t.fill_(POISON_I32)


def plan_on_gpu(layer: MoEProjection, topk_np):
    topk = torch.from_numpy(np.ascontiguousarray(topk_np, dtype=np.int32)).to(layer.device)
    poison_plan(layer)
    layer.plan(topk)
    torch.cuda.synchronize()
    c = layer.cfg
    N = c.R * c.S
    return dict(
        cu_seqlens=layer.cu_seqlens.cpu().numpy(),
        replica_expert=layer.replica_expert[:, :c.B].cpu().numpy(),
        slot_map=layer.slot_map[:N * c.K].cpu().numpy(),
        src_index=layer.src_index[:N * c.K].cpu().numpy(),
    ), topk


def assert_plan_equal(got, pl):
    for name in ("cu_seqlens", "replica_expert", "slot_map", "src_index"):
        want = getattr(pl, name)
        g = got[name]
        assert g.shape == want.shape, (name, g.shape, want.shape)
        if not np.array_equal(g, want):
            bad = np.argwhere(g != want)
            raise AssertionError(f"{name} differs at {len(bad)} places, first {bad[:5].tolist()}: "
                                 f"got {g[tuple(bad[0])]} want {want[tuple(bad[0])]}")


def rel_err(got, ref):
    """max |got - ref| / RMS(ref)."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.abs(np.asarray(got, dtype=np.float64) - ref).max() / max(rms, 1e-300))


def tolerance(cfg) -> float:
    # max abs error <= 1e-2 * RMS(reference) for bf16 layers, 1e-5 * RMS for fp32
    return 1e-2 if cfg.dtype == "bf16" else 1e-5


def assert_stored_close(got, ref, dtype, what=""):
    """An intermediate the layer stores in its dtype (the SwiGLU output, the saved
    pre-activation), element by element: within one rounding step of the stored
    type of the oracle's value (2^-7 relative for bfloat16, 2^-22 for float32) plus
    the float32 accumulation-order error upstream of the rounding, which shows where
    the value is near zero (1e-4 * RMS(ref) for bfloat16 layers, whose bar is
    1e-2 * RMS; 1e-5 * RMS for float32 layers).
    (A max-abs / RMS bound does not fit such tensors: where the float32 and the
    float64 sums straddle a rounding boundary the stored value moves by a whole
    step of that element, and the largest elements are many RMS.)"""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    step = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -22
    rms = np.sqrt(np.mean(ref * ref))
    floor = 1e-4 if dtype == "bf16" else 1e-5
    bad = np.abs(got - ref) > step * np.abs(ref) + floor * rms
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements off, first at {i}: "
                             f"got {got[i]!r} want {ref[i]!r} (RMS {rms:.4g})")
