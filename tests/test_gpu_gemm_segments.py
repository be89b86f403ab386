"""Grouped GEMM on hand-made cu_seqlens whose segment lengths sit on every tile boundary
(1, 15-17, 63-65, 127-129, 191-193, 255-257, 383-385, 511-513 rows), compared in full
with the oracle's segment_matmul and segment_wgrad [the hot path's rows:
ai-maestro.online "Moonshot AI open-sources MoonEP", section "The memory contract": the
group GEMM addresses experts by row index and cu_seqlens selects the rows].

Two sizes, every op (FWD, DGRAD, WGRAD):
* at least four rounds of full 256 x 256 tiles over the compute units: the forward takes
  the per-XCD tile queues and runs each last tile of at most 128 rows with the tile's
  second row group idle; DGRAD sends those tiles to the 128 x 512 tail launch;
* a small call on 128 x 128 tiles, whose second row group idles on last tiles of at most
  64 rows.
Each rank's segments lie in its home rows and its prefetch slots, as a training plan's
do (WGRAD's precondition); one such row per rank stays empty. Outputs are poisoned with
NaN (FWD, DGRAD) or start from seeded values (WGRAD's += targets). Tolerance as
elsewhere: max abs error <= 1e-2 * RMS(reference) for bfloat16.
"""
import numpy as np
import pytest
import torch

from oracle import moe as M
from redundant_expert_balancing_amd import _lib as L

from gpu_helpers import rel_err, say, small_cfg

pytestmark = pytest.mark.gpu

BOUNDARY = [1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257,
            383, 384, 385, 511, 512, 513]
TILE_M = 256


def _cu_seqlens(R, E, B, SK, rng):
    """Per rank: boundary lengths (a rotating share of BOUNDARY) on its home rows and
    slots, one of those rows empty, the rest of the S*K slots spread over the others."""
    G = E // R
    cu = np.zeros((R, E + B + 1), dtype=np.int32)
    per = -(-len(BOUNDARY) // R) + 6
    for q in range(R):
        rows = rng.permutation(np.r_[np.arange(q * G, (q + 1) * G), np.arange(E, E + B)])
        lens = np.zeros(E + B, dtype=np.int64)
        take = [BOUNDARY[(q * 5 + j) % len(BOUNDARY)] for j in range(per)]
        for r, n in zip(rows[1:], take):
            lens[r] = n
        fill = rows[1 + per:]
        left = SK - int(lens.sum())
        assert left >= len(fill) and len(fill) > 0
        lens[fill] = 1 + rng.multinomial(left - len(fill), np.ones(len(fill)) / len(fill))
        cu[q, 1:] = np.cumsum(lens)
        assert cu[q, -1] == SK and lens[rows[0]] == 0
    return cu


def _randn(gen, shape, scale=1.0):
    """Seeded N(0, scale^2) float32 values drawn on the device."""
    return torch.randn(shape, generator=gen, device="cuda") * scale


def _host(t):
    return t.float().cpu().numpy()


@pytest.mark.parametrize("S", [4096, 512], ids=["large", "small_call"])
def test_gemm_on_boundary_segments_full_compare(S):
    R, E, K, H, Hp = 8, 64, 8, 128, 256
    cfg = small_cfg(name=f"segments_S{S}", R=R, S=S, E=E, K=K, H=H, Hp=Hp)
    B, SK = cfg.B, S * K
    sh = L.Shape.of(cfg)
    rng = np.random.default_rng(S)
    cu = _cu_seqlens(R, E, B, SK, rng)
    n = np.diff(cu, axis=1).ravel()
    n = n[n > 0]
    last = n - (n - 1) // TILE_M * TILE_M
    say("segments", S, "non-empty", len(n), "last tiles <=128 rows", int((last <= 128).sum()))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    full_tiles = R * SK // TILE_M
    if S == 4096:
        assert full_tiles >= 4 * cus        # tails treated apart, queued forward
    else:
        assert full_tiles < 2 * cus         # small call: 128 x 128 tiles
    dev = torch.device("cuda")
    gen = torch.Generator(device="cuda").manual_seed(S)
    xp = _randn(gen, (R * SK, H)).to(torch.bfloat16)
    dyp = _randn(gen, (R * SK, Hp)).to(torch.bfloat16)
    w_all = _randn(gen, (E + R * B, H, Hp), H ** -0.5).to(torch.bfloat16)
    cu_d = torch.from_numpy(cu).to(dev)
    ws = torch.empty((L.moonep_workspace_bytes(sh) // 4,), dtype=torch.int32, device=dev)
    L.moonep_workspace_init(sh, ws)
    out = torch.full((R * SK, Hp), float("nan"), device=dev)
    dxp = torch.full((R * SK, H), float("nan"), device=dev)
    g0 = _randn(gen, (E, H, Hp))
    r0 = _randn(gen, (R, B, H, Hp))
    grad_home, reduce_buf = g0.clone(), r0.clone()
    say("gemm FWD, DGRAD, WGRAD", S)
    L.moonep_grouped_gemm(sh, L.FWD, xp, w_all, cu_d, out, None, None, ws)
    L.moonep_grouped_gemm(sh, L.DGRAD, dyp, w_all, cu_d, dxp, None, None, ws)
    L.moonep_grouped_gemm(sh, L.WGRAD, xp, dyp, cu_d, None, grad_home, reduce_buf, ws)
    torch.cuda.synchronize()
    assert L.moonep_get_error(sh, ws) == 0

    xp_h, dyp_h, w_h = _host(xp), _host(dyp), _host(w_all)
    out_ref = M.segment_matmul(xp_h, w_h, cu, R, SK, E, B)
    e_out = rel_err(_host(out), out_ref)
    dxp_ref = M.segment_matmul(dyp_h, w_h, cu, R, SK, E, B, transpose_w=True)
    e_dxp = rel_err(_host(dxp), dxp_ref)
    gh = g0.cpu().numpy().astype(np.float64)
    rb = r0.cpu().numpy().astype(np.float64)
    M.segment_wgrad(xp_h, dyp_h, cu, R, SK, E, B, gh, rb)
    e_gh = rel_err(grad_home.cpu().numpy(), gh)
    e_rb = rel_err(reduce_buf.cpu().numpy(), rb)
    say("segments", S, "out", e_out, "dxp", e_dxp, "grad_home", e_gh, "reduce_buf", e_rb)
    assert max(e_out, e_dxp, e_gh, e_rb) <= 1e-2
