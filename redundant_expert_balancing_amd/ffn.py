"""Device buffers of the full expert FFN of an R-rank MoE layer held on one GPU,
and its hot path as a sequence of library calls (no computation here).

One plan serves both projections [ai-maestro.online "Moonshot AI open-sources
MoonEP", section "The memory contract": the weight contract is per projection,
[E+B, H, H'] per expert weight]:

Forward  : plan -> prefetch(W1, W2) -> dispatch(x) -> gate/up GEMM with SwiGLU
           -> down GEMM -> combine(z, gates)
Backward : dispatch(dy, gates) -> dgrad(W2) -> wgrad(W2) -> SwiGLU backward
           -> dgrad(W1) -> wgrad(W1) -> combine(dxp, no gates) -> reduce_grad(W1, W2)

Shapes passed to the library (H' = cfg.Hp, the intermediate size):
  ffn  (H, H')    SwiGLU calls        up  (H, 2H')   everything on W1, x, dX
  down (H', H)    everything on W2, the down projection's output z
Buffer layout (row-major, one allocation per array; rows = R*S*K):
  w1_all dtype [E+R*B, H, 2H'] (gate/up columns interleaved in 32-column blocks)
  w2_all dtype [E+R*B, H', H];  xp dtype [rows, H];  act dtype [rows, H']
  h fp32 [rows, 2H'] (unfused path only);  hs dtype [rows, 2H'] (training)
  z fp32 [rows, H];  y fp32 [N, H]
  backward: dyp dtype [rows, H]; da fp32 [rows, H']; dh dtype [rows, 2H'];
  dxp fp32 [rows, H]; dx fp32 [N, H]; grad1 fp32 [E, H, 2H']; red1 fp32
  [R, B, H, 2H']; grad2 fp32 [E, H', H]; red2 fp32 [R, B, H', H]
"""
from __future__ import annotations

import torch

from . import _lib as L


def _shape(cfg, H, Hp):
    return L.Shape(cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, H, Hp,
                   L.TRAIN if cfg.mode == "train" else L.INFER,
                   L.BF16 if cfg.dtype == "bf16" else L.FP32)


class MoEFFN:
    def __init__(self, cfg, device="cuda", backward: bool = False, w1_all=None, w2_all=None,
                 fused: bool = True):
        c = cfg
        self.cfg = c
        self.fused = fused
        self.shape = _shape(c, c.H, c.Hp)
        self.up = _shape(c, c.H, 2 * c.Hp)
        self.down = _shape(c, c.Hp, c.H)
        for sh in (self.shape, self.up, self.down):
            st = L.moonep_validate_shape(sh)
            if st != L.OK:
                raise L.MoonepError("moonep_validate_shape", st)
        if c.H % 64 or c.Hp % 64:
            raise L.MoonepError("MoEFFN (H and H' must be multiples of 64)", L.EINVAL)
        self.device = torch.device(device)
        dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        self.dtype = dt
        N, rows = c.R * c.S, max(c.R * c.S * c.K, 1)
        i32 = dict(dtype=torch.int32, device=self.device)
        f32 = dict(dtype=torch.float32, device=self.device)
        dtd = dict(dtype=dt, device=self.device)
        self.cu_seqlens = torch.empty((c.R, c.E + c.B + 1), **i32)
        self.replica_expert = torch.empty((c.R, max(c.B, 1)), **i32)
        self.slot_map = torch.empty((max(N * c.K, 1),), **i32)
        self.src_index = torch.empty((max(N * c.K, 1),), **i32)
        self.ws = torch.empty((L.moonep_workspace_bytes(self.up) // 4,), **i32)
        L.moonep_workspace_init(self.up, self.ws)
        W = c.E + c.R * c.B
        self.w1_all = w1_all if w1_all is not None else torch.empty((W, c.H, 2 * c.Hp), **dtd)
        self.w2_all = w2_all if w2_all is not None else torch.empty((W, c.Hp, c.H), **dtd)
        self.xp = torch.empty((rows, c.H), **dtd)
        self.act = torch.empty((rows, c.Hp), **dtd)
        self.h = None if fused else torch.empty((rows, 2 * c.Hp), **f32)
        self.hs = torch.empty((rows, 2 * c.Hp), **dtd) if backward else None
        self.z = torch.empty((rows, c.H), **f32)
        self.y = torch.empty((max(N, 1), c.H), **f32)
        if backward:
            self.dyp = torch.empty((rows, c.H), **dtd)
            self.da = torch.empty((rows, c.Hp), **f32)
            self.dh = torch.empty((rows, 2 * c.Hp), **dtd)
            self.dxp = torch.empty((rows, c.H), **f32)
            self.dx = torch.empty((max(N, 1), c.H), **f32)
            B = max(c.B, 1)
            self.grad1 = torch.zeros((c.E, c.H, 2 * c.Hp), **f32)
            self.red1 = torch.zeros((c.R, B, c.H, 2 * c.Hp), **f32)
            self.grad2 = torch.zeros((c.E, c.Hp, c.H), **f32)
            self.red2 = torch.zeros((c.R, B, c.Hp, c.H), **f32)

    # ---- forward stages
    def plan(self, topk_idx, stream=None):
        L.moonep_plan(self.up, topk_idx, self.cu_seqlens, self.replica_expert, self.slot_map,
                      self.src_index, self.ws, stream)

    def prefetch(self, stream=None):
        L.moonep_prefetch_weight(self.up, self.replica_expert, self.w1_all, stream)
        L.moonep_prefetch_weight(self.down, self.replica_expert, self.w2_all, stream)

    def dispatch(self, x, stream=None):
        L.moonep_dispatch(self.up, self.cfg.H, x, self.slot_map, None, self.xp, stream)

    def gate_up(self, stream=None):
        if self.fused:
            L.moonep_grouped_gemm_swiglu(self.shape, self.xp, self.w1_all, self.cu_seqlens,
                                         self.act, self.hs, self.ws, stream)
        else:
            L.moonep_grouped_gemm(self.up, L.FWD, self.xp, self.w1_all, self.cu_seqlens, self.h,
                                  None, None, self.ws, stream)
            L.moonep_swiglu(self.shape, self.h, self.act, self.hs, stream)

    def down_proj(self, stream=None):
        L.moonep_grouped_gemm(self.down, L.FWD, self.act, self.w2_all, self.cu_seqlens, self.z,
                              None, None, self.ws, stream)

    def combine(self, gates, stream=None):
        L.moonep_combine(self.up, self.cfg.H, self.z, self.slot_map, gates, self.y, stream)

    def forward(self, topk_idx, x, gates, stream=None):
        self.plan(topk_idx, stream)
        self.prefetch(stream)
        self.dispatch(x, stream)
        self.gate_up(stream)
        self.down_proj(stream)
        self.combine(gates, stream)
        return self.y

    # ---- backward
    def backward(self, dy, gates, stream=None):
        c = self.cfg
        L.moonep_dispatch(self.up, c.H, dy, self.slot_map, gates, self.dyp, stream)
        L.moonep_grouped_gemm(self.down, L.DGRAD, self.dyp, self.w2_all, self.cu_seqlens, self.da,
                              None, None, self.ws, stream)
        L.moonep_grouped_gemm(self.down, L.WGRAD, self.act, self.dyp, self.cu_seqlens, None,
                              self.grad2, self.red2, self.ws, stream)
        L.moonep_swiglu_backward(self.shape, self.hs, self.da, self.dh, stream)
        L.moonep_grouped_gemm(self.up, L.DGRAD, self.dh, self.w1_all, self.cu_seqlens, self.dxp,
                              None, None, self.ws, stream)
        L.moonep_grouped_gemm(self.up, L.WGRAD, self.xp, self.dh, self.cu_seqlens, None,
                              self.grad1, self.red1, self.ws, stream)
        L.moonep_combine(self.up, c.H, self.dxp, self.slot_map, None, self.dx, stream)
        L.moonep_reduce_grad(self.up, self.replica_expert, self.red1, self.grad1, stream)
        L.moonep_reduce_grad(self.down, self.replica_expert, self.red2, self.grad2, stream)
        return self.dx

    def error_flags(self, clear=False) -> int:
        return L.moonep_get_error(self.up, self.ws, clear)
