"""Device buffers of one expert projection of an R-rank MoE layer held on one GPU,
and the hot path as a sequence of library calls (no computation here).

Forward  : plan -> prefetch_weight -> dispatch(x) -> grouped_gemm(FWD) -> combine(out, gates)
Backward : dispatch(dy, gates) -> grouped_gemm(DGRAD) -> grouped_gemm(WGRAD)
           -> combine(dxp, no gates) -> reduce_grad
Buffer layout (row-major, one allocation per array):
  topk_idx int32 [N,K]; gates fp32 [N,K]; cu_seqlens int32 [R,E+B+1];
  replica_expert int32 [R,B]; slot_map, src_index int32 [N*K];
  w_all dtype [E+R*B,H,H'] (home rows, then each rank's prefetch slots);
  xp dtype [R*SK,H]; out fp32 [R*SK,H']; y fp32 [N,H'];
  dyp dtype [R*SK,H']; dxp fp32 [R*SK,H]; dx fp32 [N,H];
  grad_home fp32 [E,H,H']; reduce_buf fp32 [R,B,H,H'].
"""
from __future__ import annotations

import torch

from . import _lib as L


class MoEProjection:
    def __init__(self, cfg, device="cuda", backward: bool = False, w_all=None):
        self.cfg = cfg
        self.shape = L.Shape.of(cfg)
        st = L.moonep_validate_shape(self.shape)
        if st != L.OK:
            raise L.MoonepError("moonep_validate_shape", st)
        self.device = torch.device(device)
        c = cfg
        dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        self.dtype = dt
        N, SK = c.R * c.S, c.S * c.K
        i32 = dict(dtype=torch.int32, device=self.device)
        self.cu_seqlens = torch.empty((c.R, c.E + c.B + 1), **i32)
        self.replica_expert = torch.empty((c.R, max(c.B, 1)), **i32)
        self.slot_map = torch.empty((max(N * c.K, 1),), **i32)
        self.src_index = torch.empty((max(N * c.K, 1),), **i32)
        self.ws = torch.empty((L.moonep_workspace_bytes(self.shape) // 4,), **i32)
        L.moonep_workspace_init(self.shape, self.ws)
        if w_all is None:
            w_all = torch.empty((c.E + c.R * c.B, c.H, c.Hp), dtype=dt, device=self.device)
        self.w_all = w_all
        self.xp = torch.empty((max(c.R * SK, 1), c.H), dtype=dt, device=self.device)
        self.out = torch.empty((max(c.R * SK, 1), c.Hp), dtype=torch.float32, device=self.device)
        self.y = torch.empty((max(N, 1), c.Hp), dtype=torch.float32, device=self.device)
        if backward:
            self.dyp = torch.empty((max(c.R * SK, 1), c.Hp), dtype=dt, device=self.device)
            self.dxp = torch.empty((max(c.R * SK, 1), c.H), dtype=torch.float32, device=self.device)
            self.dx = torch.empty((max(N, 1), c.H), dtype=torch.float32, device=self.device)
            self.grad_home = torch.zeros((c.E, c.H, c.Hp), dtype=torch.float32, device=self.device)
            self.reduce_buf = torch.zeros((c.R, max(c.B, 1), c.H, c.Hp), dtype=torch.float32,
                                          device=self.device)

    # ---- stages
    def plan(self, topk_idx, stream=None):
        L.moonep_plan(self.shape, topk_idx, self.cu_seqlens, self.replica_expert, self.slot_map,
                      self.src_index, self.ws, stream)

    def prefetch(self, stream=None):
        L.moonep_prefetch_weight(self.shape, self.replica_expert, self.w_all, stream)

    def dispatch(self, x, stream=None):
        L.moonep_dispatch(self.shape, self.cfg.H, x, self.slot_map, None, self.xp, stream)

    def gemm_fwd(self, stream=None):
        L.moonep_grouped_gemm(self.shape, L.FWD, self.xp, self.w_all, self.cu_seqlens, self.out,
                              None, None, self.ws, stream)

    def combine(self, gates, stream=None):
        L.moonep_combine(self.shape, self.cfg.Hp, self.out, self.slot_map, gates, self.y, stream)

    def forward(self, topk_idx, x, gates, stream=None):
        self.plan(topk_idx, stream)
        self.prefetch(stream)
        self.dispatch(x, stream)
        self.gemm_fwd(stream)
        self.combine(gates, stream)
        return self.y

    def backward(self, dy, gates, stream=None):
        c = self.cfg
        L.moonep_dispatch(self.shape, c.Hp, dy, self.slot_map, gates, self.dyp, stream)
        L.moonep_grouped_gemm(self.shape, L.DGRAD, self.dyp, self.w_all, self.cu_seqlens,
                              self.dxp, None, None, self.ws, stream)
        L.moonep_grouped_gemm(self.shape, L.WGRAD, self.xp, self.dyp, self.cu_seqlens, None,
                              self.grad_home, self.reduce_buf, self.ws, stream)
        L.moonep_combine(self.shape, c.H, self.dxp, self.slot_map, None, self.dx, stream)
        L.moonep_reduce_grad(self.shape, self.replica_expert, self.reduce_buf, self.grad_home,
                             stream)
        return self.dx

    def error_flags(self, clear=False) -> int:
        return L.moonep_get_error(self.shape, self.ws, clear)
