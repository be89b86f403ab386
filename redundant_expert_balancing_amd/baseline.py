"""Per-rank view of the grouped GEMM, and the no-redundancy (plain EP) baseline.

With real expert parallelism every rank runs its own grouped GEMM at the same
time, so the layer waits for the hottest rank [ai-maestro.online "Moonshot AI
open-sources MoonEP", sections "The problem MoonEP targets" and "Benchmarks
against DeepEP v2"]. On one GPU the R ranks share the chip, so this module cuts
one rank's share out as a one-rank grouped GEMM problem that runs on the same
kernels, to time it alone:

  balanced   rank q after the redundant-expert plan: its S*K rows over its G
             home rows and its B prefetch slots (training layers, B = G);
  home-only  plain EP without redundant experts: rank q computes every slot
             routed to its G home experts, L_q rows, whatever the skew.

The sub-problems are built with device tensor slicing only (no host sync in
the timed calls); cu_seqlens of a sub-problem is the compacted prefix of the
rank's non-empty rows.
"""
from __future__ import annotations

import torch

from . import _lib as L


def _one_rank_shape(G, S, K, B, H, Hp, mode, dtype):
    return L.Shape(1, S, G, K, B, H, Hp, L.TRAIN if mode == "train" else L.INFER,
                   L.BF16 if dtype == "bf16" else L.FP32)


class RankProblem:
    """One rank's grouped GEMM as a one-rank problem: a[rows, H] @ w[rows of cu]."""

    def __init__(self, shape, a, w, cu):
        self.shape = shape
        self.a = a
        self.w = w
        self.cu = cu
        self.out = torch.empty((a.shape[0], w.shape[2]), dtype=torch.float32, device=a.device)
        self.ws = torch.empty((L.moonep_workspace_bytes(shape) // 4,), dtype=torch.int32,
                              device=a.device)
        L.moonep_workspace_init(shape, self.ws)

    def run(self, stream=None):
        L.moonep_grouped_gemm(self.shape, L.FWD, self.a, self.w, self.cu, self.out, None, None,
                              self.ws, stream)


def balanced_rank(layer, q: int) -> RankProblem:
    """Rank q of a planned training layer: its S*K rows of xp against its home rows
    [qG, (q+1)G) followed by its B slots (contiguous copy of those weight rows)."""
    c = layer.cfg
    assert c.mode == "train" and c.B == c.G
    G, SK = c.G, c.S * c.K
    lens = torch.diff(layer.cu_seqlens[q].long())
    sel = torch.cat([lens[q * G:(q + 1) * G], lens[c.E:c.E + c.B]])
    cu = torch.zeros((1, G + c.B + 1), dtype=torch.int32, device=lens.device)
    cu[0, 1:] = torch.cumsum(sel, 0).to(torch.int32)
    w = torch.cat([layer.w_all[q * G:(q + 1) * G],
                   layer.w_all[c.E + q * c.B:c.E + (q + 1) * c.B]]).contiguous()
    shape = _one_rank_shape(G, c.S, c.K, c.B, c.H, c.Hp, "train", c.dtype)
    return RankProblem(shape, layer.xp[q * SK:(q + 1) * SK], w, cu)


def home_only_ranks(cfg, xp_sorted, cu_sorted, w_home):
    """Plain EP: rank q gets every row of its home experts out of a one-rank
    (counting-sort) plan of the whole routing: xp_sorted [N*K, H] grouped by
    expert, cu_sorted [E+1] its exclusive prefix (device). Reads the rank
    boundaries back once to size the sub-problems (set-up, not the timed call)."""
    G, K = cfg.G, cfg.K
    bounds = cu_sorted[::G].tolist()          # [R+1] row where each rank's experts start
    probs = []
    for q in range(cfg.R):
        start, rows = bounds[q], bounds[q + 1] - bounds[q]
        cu = (cu_sorted[q * G:(q + 1) * G + 1] - start).to(torch.int32).view(1, G + 1)
        S = max(1, -(-rows // K))
        shape = _one_rank_shape(G, S, K, 0, cfg.H, cfg.Hp, "infer", cfg.dtype)
        # the rank's rows, padded with zero rows to the S*K rows its shape declares
        a = torch.zeros((S * K, cfg.H), dtype=xp_sorted.dtype, device=xp_sorted.device)
        a[:rows] = xp_sorted[start:start + rows]
        probs.append(RankProblem(shape, a, w_home[q * G:(q + 1) * G].contiguous(), cu))
    return probs, [b - a for a, b in zip(bounds[:-1], bounds[1:])]
