"""A stack of MoE layers whose prefetch slots come from one process-global pool,
with the prefetches on a side stream.

[ai-maestro.online "Moonshot AI open-sources MoonEP", section "The memory
contract": the prefetch slots draw from a process-global pool shared by all
layers, so the extra memory is B expert weights per projection in total; section
"The core idea": duplicated experts are prefetched before expert computation,
and their gradients go home in the backward pass.]

Every layer's weights are a view (moonep_view_create): one contiguous
[E+R*B, H, H'] address range whose home rows are the layer's own and whose slot
rows are one set of the pool (layer l uses set l % nsets). A later layer on the
same set overwrites the replicas, so the backward pass prefetches a layer's
replicas again, from its kept plan, unless its set still holds them. The host
tracks which layer each set holds, in issue order.

Overlap (all streams at the default priority). A prefetch on the side stream
waits for an event recorded on the main stream, so it follows every earlier use
of its set there, and the main stream waits for it before the first GEMM that
reads the slots:
  forward   prefetch(l) needs plan(l), so it can overlap only dispatch(l). Both
            are HBM-bound on one GPU and share its bandwidth: measured 1.3%
            slower than serial at the bench shape, so off by default;
  backward  with two or more sets, prefetch(l-1) depends only on layer l-1's
            kept plan and writes the other set, so it is issued at the start
            of backward(l) and runs under layer l's compute-bound dgrad and
            wgrad (on by default).
This module only orders library calls; it computes nothing.
"""
from __future__ import annotations

import torch

from . import _lib as L
from .layer import MoEProjection


class _DeviceArray:
    """__cuda_array_interface__ of raw device memory, so torch can view it."""

    def __init__(self, addr: int, shape, typestr: str):
        self.__cuda_array_interface__ = {"shape": tuple(shape), "typestr": typestr,
                                         "data": (addr, False), "version": 3, "strides": None}


class SlotPool:
    """Physical prefetch-slot memory shared by every layer of one projection type."""

    def __init__(self, cfg, nsets: int = 1):
        self.cfg = cfg
        self.shape = L.Shape.of(cfg)
        self.handle = L.moonep_pool_create(self.shape, nsets)
        self.nsets = nsets

    @property
    def nbytes(self) -> int:
        return L.moonep_pool_bytes(self.handle)

    def close(self):
        if self.handle:
            L.moonep_pool_destroy(self.handle)
            self.handle = 0


class PooledWeights:
    """One layer's w_all [E+R*B, H, H'] over a pool view, as a torch tensor (it does
    not own the memory; close() unmaps it)."""

    def __init__(self, cfg, pool: SlotPool, set_index: int = 0):
        self.view, addr = L.moonep_view_create(L.Shape.of(cfg), pool.handle, set_index)
        rows = cfg.E + cfg.R * cfg.B
        if cfg.dtype == "bf16":
            raw = torch.as_tensor(_DeviceArray(addr, (rows, cfg.H, cfg.Hp), "<i2"), device="cuda")
            self.tensor = raw.view(torch.bfloat16)
        else:
            self.tensor = torch.as_tensor(_DeviceArray(addr, (rows, cfg.H, cfg.Hp), "<f4"),
                                          device="cuda")
        assert self.tensor.data_ptr() == addr

    def close(self):
        if self.view:
            self.tensor = None
            L.moonep_view_destroy(self.view)
            self.view = 0


class MoEStack:
    """n_layers projections of one shape; slots from a pool of nsets shared sets."""

    def __init__(self, cfg, n_layers: int, device="cuda", backward: bool = False,
                 nsets: int = 1, overlap_forward: bool = False, overlap_backward: bool = True):
        self.cfg = cfg
        self.overlap_forward = overlap_forward
        self.overlap_backward = overlap_backward
        self.nsets = nsets
        self.pool = SlotPool(cfg, nsets)
        self.weights = [PooledWeights(cfg, self.pool, l % nsets) for l in range(n_layers)]
        self.layers = [MoEProjection(cfg, device, backward=backward, w_all=w.tensor)
                       for w in self.weights]
        self.side = torch.cuda.Stream(device=device)
        self.holder = [-1] * nsets      # layer whose replicas each set holds (issue order)
        self.pending = {}               # layer -> event of its side-stream prefetch

    def _issue_prefetch(self, l, main, side: bool):
        layer = self.layers[l]
        self.holder[l % self.nsets] = l
        if not side:
            layer.prefetch(main)
            return
        ev = torch.cuda.Event()
        ev.record(main)                 # after every earlier use of this set on main
        self.side.wait_event(ev)
        layer.prefetch(self.side)
        done = torch.cuda.Event()
        done.record(self.side)
        self.pending[l] = done

    def _await_prefetch(self, l, main):
        ev = self.pending.pop(l, None)
        if ev is not None:
            main.wait_event(ev)

    def forward_layer(self, l, topk_idx, x, gates):
        main = torch.cuda.current_stream()
        layer = self.layers[l]
        layer.plan(topk_idx, main)
        self._issue_prefetch(l, main, self.overlap_forward)
        layer.dispatch(x, main)
        self._await_prefetch(l, main)
        layer.gemm_fwd(main)
        layer.combine(gates, main)
        return layer.y

    def backward_layer(self, l, dy, gates):
        """Layers are taken in descending order."""
        main = torch.cuda.current_stream()
        layer = self.layers[l]
        c, sh = self.cfg, layer.shape
        if self.holder[l % self.nsets] != l:
            self._issue_prefetch(l, main, self.overlap_backward)
        nxt = l - 1
        if (self.overlap_backward and nxt >= 0 and nxt % self.nsets != l % self.nsets
                and self.holder[nxt % self.nsets] != nxt):
            self._issue_prefetch(nxt, main, True)   # runs under this layer's GEMMs
        L.moonep_dispatch(sh, c.Hp, dy, layer.slot_map, gates, layer.dyp, main)
        self._await_prefetch(l, main)
        L.moonep_grouped_gemm(sh, L.DGRAD, layer.dyp, layer.w_all, layer.cu_seqlens, layer.dxp,
                              None, None, layer.ws, main)
        L.moonep_grouped_gemm(sh, L.WGRAD, layer.xp, layer.dyp, layer.cu_seqlens, None,
                              layer.grad_home, layer.reduce_buf, layer.ws, main)
        L.moonep_combine(sh, c.H, layer.dxp, layer.slot_map, None, layer.dx, main)
        L.moonep_reduce_grad(sh, layer.replica_expert, layer.reduce_buf, layer.grad_home, main)
        return layer.dx

    def close(self):
        torch.cuda.synchronize()
        self.layers = []
        for w in self.weights:
            w.close()
        self.weights = []
        self.pool.close()
