#!/usr/bin/env python3
"""Benchmark of the balanced expert-parallel MoE layer on one MI355X.

One step = one pass of the whole forward hot path over one batch of synthetic
router output at the pages' bench shape (R=8 ranks, S=8192 tokens per rank,
E=384 experts, K=8, B=48 prefetch slots, H=7168, H'=2048, bf16):
plan -> prefetch_weight -> dispatch -> grouped GEMM -> combine. Steps cycle over
the four router imbalance points maxvio in {0.2, 1, 10, 20}, all drawn from one
shared seed. Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line (rank 0). Besides the contract fields:
  roofline      the grouped GEMM (dominant kernel) against dense bf16 MFMA peak;
                its average duration comes from HIP events around every GEMM
                call inside the timed region, on the stream it runs on (one call
                = the tile-list kernel and the 256x256-tile kernel, which also
                runs the segment tails); traffic = HBM bytes of the GEMM kernel;
  cpu_baseline  the CPU oracle stage by stage (plan, permute, combine on one thread;
                the float64 dense projection on every core; the training backward of
                the training-backward layer), each on a bounded sample scaled to the
                whole layer, with the sample, thread and core counts stated;
  stages_us     per-stage median microseconds at every imbalance point
                (each repetition after a 1 GiB write that evicts the caches);
  hbm_stages    plan + dispatch + combine against the HBM peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + plan/dispatch us vs maxvio (S=8192,E=384,K=8,H=7168)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_fwd_bench_shape_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", default="bench_shape")
    ap.add_argument("--stage-reps", type=int, default=50,
                    help="timed repetitions per stage in the stage table (after 5 warm-ups)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--table", action="store_true",
                    help="only print per-stage microseconds for every layer configuration")
    ap.add_argument("--home-only-baseline", action="store_true",
                    help="only print per-rank grouped-GEMM time, balanced vs plain EP")
    ap.add_argument("--stack", type=int, default=0,
                    help="only time N layers at the bench shape whose prefetch slots share one "
                         "pool, prefetch serial vs on a side stream overlapped with dispatch")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time the vendor library's dense GEMM of the bench shape's size "
                         "(hipBLASLt through torch.mm: bf16 output, and float32 output as the "
                         "grouped GEMM writes) next to the grouped GEMM, same process and box; "
                         "a reference for the kernel, not part of the path")
    ap.add_argument("--ffn", action="store_true",
                    help="only print per-stage microseconds of the full expert FFN (gate/up "
                         "with SwiGLU, down) forward at the bench shape and backward at the "
                         "training-backward shape")
    return ap.parse_args()


def gemm_source_sha() -> str:
    with open(os.path.join(ROOT, "redundant_expert_balancing_amd", "csrc", "gemm.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic():
    """HBM bytes per GEMM launch from the committed counter runs, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha") != gemm_source_sha():
        return None
    return t.get("bytes_per_launch")


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            return next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        return "unknown"


def _compact(slot_map_part):
    """Destinations of a sample of slots renumbered 0.. in buffer order, so the oracle's
    permute and combine run on a buffer of the sample's size with the same per-slot work."""
    import numpy as np
    order = np.argsort(slot_map_part, kind="stable")
    out = np.empty_like(slot_map_part)
    out[order] = np.arange(len(slot_map_part))
    return out


def _timed(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def cpu_baseline(cfg, routing, x_dev, w_dev):
    """The oracle as it stands, stage by stage, on the host: the plan on the full routing,
    the permute and the gated combine on sampled tokens (pure-Python loops, one thread), the
    float64 dense projection on sampled tokens (BLAS on every core), and the training
    backward of the training-backward layer (gated dY permute, dense dX and dW, replica
    fold). Each sampled stage is scaled to the whole layer by its count of slots, tokens or
    consumed slots. tokens/s = N / (plan + permute + projection + combine) of the forward."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    from oracle import moe as M
    from oracle import plan as P

    cores = len(os.sched_getaffinity(0))
    N, K = cfg.N, cfg.K
    rng = np.random.default_rng(0)
    st = {}
    with threadpool_limits(1):
        t_plan = _timed(lambda: P.plan(routing.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B,
                                       cfg.mode))
        pl = P.plan(routing.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
        n_perm = 1024
        rows = x_dev[:n_perm].float().cpu().numpy()
        sm = _compact(pl.slot_map[:n_perm * K])
        t_perm = _timed(lambda: M.permute(rows, sm, K))
        n_comb = 4096
        out = rng.standard_normal((n_comb * K, cfg.Hp)).astype(np.float32)
        smc = _compact(pl.slot_map[:n_comb * K])
        t_comb = _timed(lambda: M.combine(out, smc, routing.gates[:n_comb], n_comb, K))
    st["plan"] = {"s": round(t_plan, 3), "sample": f"full routing, {N * K} slots", "threads": 1}
    st["permute"] = {"s": round(t_perm * N / n_perm, 2), "sample_s": round(t_perm, 3),
                     "sample": f"{n_perm} tokens ({n_perm * K} slots)", "threads": 1}
    st["combine"] = {"s": round(t_comb * N / n_comb, 2), "sample_s": round(t_comb, 3),
                     "sample": f"{n_comb} tokens", "threads": 1}
    # float64 dense projection on every core; the sample touches every expert, so each
    # expert's weight conversion is amortised as over the whole batch
    n_tok = min(N, 2 * cfg.S)
    toks = np.sort(rng.choice(N, n_tok, replace=False))
    x_s = x_dev[torch.from_numpy(toks).cuda()].float().cpu().numpy()
    experts = np.unique(routing.topk_idx[toks])
    W = {int(e): w_dev[int(e)].float().cpu().numpy() for e in experts}   # inputs, fetched first

    class Wmap:
        shape = (cfg.E, cfg.H, cfg.Hp)

        def __getitem__(self, e):
            return W[int(e)]

    t_dense = _timed(lambda: M.dense_forward(x_s, Wmap(), routing.topk_idx[toks],
                                             routing.gates[toks]))
    del W
    st["projection"] = {"s": round(t_dense * N / n_tok, 2), "sample_s": round(t_dense, 3),
                        "sample": f"{n_tok} tokens", "threads": cores}
    fwd = sum(st[k]["s"] for k in ("plan", "permute", "projection", "combine"))
    bwd = cpu_baseline_backward(cores)
    return {"value": round(N / fwd, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": (f"forward at {cfg.name} maxvio {routing.maxvio:.3g}: plan on the full "
                       f"routing, permute / combine / dense projection on {n_perm} / {n_comb} / "
                       f"{n_tok} sampled tokens, each scaled to the {N}-token layer; plan, "
                       f"permute and combine on 1 thread, the projection on {cores}"),
            "stages_s": st, "forward_s": round(fwd, 2), "train_backward": bwd}


def cpu_baseline_backward(cores):
    """The oracle's training backward at the training-backward layer: gated permute of dY
    and unpermute of dX (1 thread) on sampled tokens, dense dX and dW (every core) on
    sampled tokens, and the replica fold (reduce_grad) on two consumed slots, each scaled to
    the whole layer."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    from oracle import moe as M
    from oracle import plan as P
    from redundant_expert_balancing_amd.synth import CONFIGS, make_dense, make_routing

    cfg = CONFIGS["train_backward"]
    r = make_routing(cfg, 15.0)
    pl = P.plan(r.topk_idx, cfg.R, cfg.S, cfg.E, cfg.K, cfg.B, cfg.mode)
    d = make_dense(cfg, "cuda", 0, which=("x", "W", "dy"))
    N, K = cfg.N, cfg.K
    rng = np.random.default_rng(1)
    st = {}
    n_perm, n_comb = 256, 4096
    dy_h = d["dy"][:max(n_perm, 1)].float().cpu().numpy()
    with threadpool_limits(1):
        t_g = _timed(lambda: M.permute(M.gated_dy(dy_h[:n_perm], r.gates[:n_perm], cfg.dtype),
                                       _compact(pl.slot_map[:n_perm * K]), K, per_slot=True))
        dxp = rng.standard_normal((n_comb * K, cfg.H)).astype(np.float32)
        smc = _compact(pl.slot_map[:n_comb * K])
        t_u = _timed(lambda: M.combine(dxp, smc, None, n_comb, K))
    st["gated_dy_permute"] = {"s": round(t_g * N / n_perm, 2), "sample_s": round(t_g, 3),
                              "sample": f"{n_perm} tokens", "threads": 1}
    st["unpermute_dx"] = {"s": round(t_u * N / n_comb, 2), "sample_s": round(t_u, 3),
                          "sample": f"{n_comb} tokens", "threads": 1}
    n_tok = 1024
    toks = np.sort(rng.choice(N, n_tok, replace=False))
    tk = torch.from_numpy(toks).cuda()
    x_s = d["x"][tk].float().cpu().numpy()
    dd = M.gated_dy(d["dy"][tk].float().cpu().numpy(), r.gates[toks], cfg.dtype)
    W = d["W"].float().cpu().numpy()                                     # inputs, fetched first
    t_d = _timed(lambda: M.dense_backward(x_s, W, r.topk_idx[toks], dd))
    del W
    st["dense_dx_dw"] = {"s": round(t_d * N / n_tok, 2), "sample_s": round(t_d, 3),
                         "sample": f"{n_tok} tokens", "threads": cores}
    consumed = int((pl.replica_expert >= 0).sum())
    rep = np.array([[0, 1]], dtype=np.int32)
    gh = rng.standard_normal((2, cfg.H, cfg.Hp))
    rb = rng.standard_normal((1, 2, cfg.H, cfg.Hp))
    with threadpool_limits(1):
        t_f = _timed(lambda: M.reduce_grad(rep, rb, gh))
    st["reduce_grad"] = {"s": round(t_f * consumed / 2, 3), "sample_s": round(t_f, 3),
                         "sample": f"2 of {consumed} consumed slots", "threads": 1}
    total = sum(v["s"] for v in st.values())
    return {"layer": cfg.name, "maxvio": round(r.maxvio, 3), "stages_s": st, "total_s": round(total, 2),
            "tokens_per_s": round(N / total, 3)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the R expert-parallel ranks are emulated as "
              "partitions of one GPU's memory, so --gpus above 1 is not supported.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from redundant_expert_balancing_amd import _lib as L
    from redundant_expert_balancing_amd.layer import MoEProjection
    from redundant_expert_balancing_amd.synth import CONFIGS, make_dense, make_routing

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.table:
        all_configs_table(args.stage_reps)
        return
    if args.home_only_baseline:
        home_only_baseline(args.stage_reps)
        return
    if args.ffn:
        ffn_table(args.stage_reps)
        return
    if args.vendor_gemm:
        vendor_gemm(args.stage_reps)
        return
    if args.stack:
        stack_bench(args.stack, args.steps, args.warmup)
        return
    L.lib()   # fail loudly if the HIP library is missing

    cfg = CONFIGS[args.config]
    print(f"[bench] {cfg.name}: generating routing for maxvio {cfg.maxvio}", file=sys.stderr, flush=True)
    routings = [make_routing(cfg, t) for t in cfg.maxvio]
    d = make_dense(cfg, "cuda", 0, which=("x", "W"), w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEProjection(cfg, "cuda", w_all=d["W"])
    x = d["x"]
    topks = [torch.from_numpy(r.topk_idx).cuda() for r in routings]
    gates = [torch.from_numpy(r.gates).cuda() for r in routings]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    N = cfg.N
    n_pts = len(routings)

    def step(i, ev=None):
        j = i % n_pts
        layer.plan(topks[j])
        layer.prefetch()
        layer.dispatch(x)
        if ev is not None:
            ev[0].record(stream)
        layer.gemm_fwd()
        if ev is not None:
            ev[1].record(stream)
        layer.combine(gates[j])

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    gemm_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(i, gemm_ev[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    gemm_ms = float(np.mean([a.elapsed_time(b) for a, b in gemm_ev]))
    assert layer.error_flags() == 0

    flops = 2.0 * cfg.H * cfg.Hp * N * cfg.K
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic(),
                "kernel": "moonep_grouped_gemm FWD: gemm_bf16_kernel 256x256 tiles (segment tails included)",
                "avg_launch_ms": round(gemm_ms, 4), "flop_per_launch": flops}

    out = {
        "metric": METRIC,
        "value": round(N * args.steps / (ms_total * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "R": cfg.R, "S": cfg.S, "E": cfg.E, "K": cfg.K,
                   "B": cfg.B, "H": cfg.H, "Hp": cfg.Hp, "maxvio": list(cfg.maxvio),
                   "mode": cfg.mode, "parallelism": f"ep{cfg.R} emulated on 1 GPU"},
        "roofline": roofline,
        "wall_s": round(wall, 3),
    }

    if not args.no_stages:
        out["stages_us"], out["hbm_stages"] = stage_table(cfg, layer, x, topks, gates, routings,
                                                          args.stage_reps)
        out["tokens_per_s_excluding_prefetch"] = tokens_excluding_prefetch(cfg, out["stages_us"])
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, routings[-1], x, d["W"])
    print(json.dumps(out), flush=True)


def stage_table(cfg, layer, x, topks, gates, routings, reps, warm=5):
    """Median (and minimum, key suffix _min) microseconds of each stage per imbalance
    point over `reps` repetitions after `warm` untimed ones, each repetition after a
    1 GiB write that evicts the caches."""
    import numpy as np
    import torch

    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    stages = {
        "plan": lambda j: layer.plan(topks[j]),
        "prefetch": lambda j: layer.prefetch(),
        "dispatch": lambda j: layer.dispatch(x),
        "gemm": lambda j: layer.gemm_fwd(),
        "combine": lambda j: layer.combine(gates[j]),
    }
    table = {}
    for j, r in enumerate(routings):
        layer.plan(topks[j])
        layer.prefetch()
        layer.dispatch(x)
        layer.gemm_fwd()
        row = {}
        for name, fn in stages.items():
            for _ in range(warm):
                fn(j)
            ts = []
            for _ in range(reps):
                flush.fill_(1.0)
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn(j)
                b.record(stream)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3)
            row[name] = round(float(np.median(ts)), 1)
            row[name + "_min"] = round(float(np.min(ts)), 1)
        row["replicas"] = int((layer.replica_expert[:, :cfg.B] >= 0).sum())
        # the skew the plan removes: the hottest rank's home load over S*K
        T = np.bincount(r.topk_idx.ravel(), minlength=cfg.E)
        row["max_home_load_over_SK"] = round(float(T.reshape(cfg.R, cfg.G).sum(1).max())
                                             / (cfg.S * cfg.K), 4)
        table[f"maxvio={r.maxvio:.3g}"] = row
    N, K, H, Hp = cfg.N, cfg.K, cfg.H, cfg.Hp
    plan_b = 12 * N * K + 4 * cfg.R * (cfg.E + cfg.B + 1)
    disp_b = N * H * 2 + N * K * H * 2 + 4 * N * K
    comb_b = N * K * Hp * 4 + 8 * N * K + N * Hp * 4
    t = float(np.mean([v["plan"] + v["dispatch"] + v["combine"] for v in table.values()]))
    gbs = (plan_b + disp_b + comb_b) / (t * 1e-6) / 1e9
    hbm = {"bytes": plan_b + disp_b + comb_b, "us": round(t, 1), "achieved": round(gbs, 1),
           "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    return table, hbm


def tokens_excluding_prefetch(cfg, table):
    """The second figure of the metric: R*S / (plan + dispatch + GEMM + combine), stage
    medians averaged over the imbalance points (prefetch scales with the replica count
    by construction and is left out)."""
    import numpy as np
    t = float(np.mean([v["plan"] + v["dispatch"] + v["gemm"] + v["combine"]
                       for v in table.values()]))
    return round(cfg.N / (t * 1e-6), 1)


def all_configs_table(reps):
    """Median microseconds per stage (caches flushed before each repetition) for
    every layer configuration and imbalance point; backward stages where the
    layer trains with backward."""
    import numpy as np
    import torch

    from redundant_expert_balancing_amd.layer import MoEProjection
    from redundant_expert_balancing_amd.synth import CONFIGS, make_dense, make_routing

    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

    def timed(fn):
        ts = []
        for _ in range(reps):
            flush.fill_(1.0)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        return round(float(np.median(ts)), 1)

    out = {}
    for name, cfg in CONFIGS.items():
        d = make_dense(cfg, "cuda", 0, which=("x", "W", "dy") if cfg.backward else ("x", "W"),
                       w_rows=cfg.E + cfg.R * cfg.B)
        layer = MoEProjection(cfg, "cuda", backward=cfg.backward, w_all=d["W"])
        for target in cfg.maxvio:
            r = make_routing(cfg, target)
            topk = torch.from_numpy(r.topk_idx).cuda()
            gates = torch.from_numpy(r.gates).cuda()
            layer.forward(topk, d["x"], gates)
            row = {"plan": timed(lambda: layer.plan(topk)),
                   "prefetch": timed(layer.prefetch),
                   "dispatch": timed(lambda: layer.dispatch(d["x"])),
                   "gemm": timed(layer.gemm_fwd),
                   "combine": timed(lambda: layer.combine(gates))}
            if cfg.backward:
                from redundant_expert_balancing_amd import _lib as L
                sh = layer.shape
                row["dispatch_dy"] = timed(lambda: L.moonep_dispatch(sh, cfg.Hp, d["dy"], layer.slot_map, gates, layer.dyp))
                row["dgrad"] = timed(lambda: L.moonep_grouped_gemm(sh, L.DGRAD, layer.dyp, layer.w_all, layer.cu_seqlens, layer.dxp, None, None, layer.ws))
                row["wgrad"] = timed(lambda: L.moonep_grouped_gemm(sh, L.WGRAD, layer.xp, layer.dyp, layer.cu_seqlens, None, layer.grad_home, layer.reduce_buf, layer.ws))
                row["unpermute"] = timed(lambda: L.moonep_combine(sh, cfg.H, layer.dxp, layer.slot_map, None, layer.dx))
                row["reduce_grad"] = timed(lambda: L.moonep_reduce_grad(sh, layer.replica_expert, layer.reduce_buf, layer.grad_home))
            row["replicas"] = int((layer.replica_expert[:, :cfg.B] >= 0).sum()) if cfg.B else 0
            out[f"{name} maxvio={r.maxvio:.3g}"] = row
            print(f"[table] {name} {target}: {row}", file=sys.stderr, flush=True)
        del layer, d
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def home_only_baseline(reps):
    """Per-rank grouped-GEMM time at the bench shape, as if every rank ran on its
    own GPU: the balanced plan (S*K rows per rank) against plain EP without
    redundant experts (rank q computes all L_q rows of its home experts). The
    layer waits for the slowest rank, so the max over ranks is the layer time."""
    import numpy as np
    import torch

    from redundant_expert_balancing_amd.baseline import balanced_rank, home_only_ranks
    from redundant_expert_balancing_amd.layer import MoEProjection
    from redundant_expert_balancing_amd.synth import CONFIGS, LayerConfig, make_dense, make_routing

    cfg = CONFIGS["bench_shape"]
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

    def timed(fn):
        ts = []
        for _ in range(reps):
            flush.fill_(1.0)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        return float(np.median(ts))

    d = make_dense(cfg, "cuda", 0, which=("x", "W"), w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEProjection(cfg, "cuda", w_all=d["W"])
    one = LayerConfig("one_rank", 1, cfg.N, cfg.E, cfg.K, 0, cfg.H, cfg.Hp, cfg.dtype, "infer",
                      cfg.maxvio)
    layer1 = MoEProjection(one, "cuda", w_all=d["W"][:cfg.E])
    out = {}
    for target in cfg.maxvio:
        r = make_routing(cfg, target)
        topk = torch.from_numpy(r.topk_idx).cuda()
        gates = torch.from_numpy(r.gates).cuda()
        layer.forward(topk, d["x"], gates)
        layer1.plan(topk)
        layer1.dispatch(d["x"])
        torch.cuda.synchronize()
        bal = []
        for q in range(cfg.R):
            p = balanced_rank(layer, q)
            bal.append(timed(p.run))
            del p
        probs, rows = home_only_ranks(cfg, layer1.xp, layer1.cu_seqlens[0], d["W"])
        home = [timed(p.run) for p in probs]
        del probs
        SK = cfg.S * cfg.K
        row = {"balanced_rank_us_max": round(max(bal), 1), "balanced_rank_us_mean": round(float(np.mean(bal)), 1),
               "plain_ep_rank_us_max": round(max(home), 1), "plain_ep_rank_us_mean": round(float(np.mean(home)), 1),
               "hottest_rank_rows_over_SK": round(max(rows) / SK, 4),
               "slowdown_plain_over_balanced": round(max(home) / max(bal), 3)}
        out[f"maxvio={r.maxvio:.3g}"] = row
        print(f"[home-only] {target}: {row}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def _timer(reps):
    """Median microseconds of fn over reps runs, each after a 1 GiB write that
    evicts the caches, timed with HIP events on the current stream."""
    import numpy as np
    import torch

    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

    def timed(fn):
        ts = []
        for _ in range(reps):
            flush.fill_(1.0)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        return round(float(np.median(ts)), 1)
    return timed


def stack_bench(n_layers, steps, warmup):
    """Layers whose slots come from one process-global pool.

    Forward, bench shape: n_layers layers (own weights and router output, the
    imbalance points in turn), one slot set, the prefetch on the main stream or
    on a side stream overlapped with dispatch.
    Backward, training-backward shape: the stack's backward with one set and the
    prefetches serial, against two sets with the next layer's prefetch on the side
    stream under the current layer's GEMMs.
    Milliseconds per layer (median of ``steps`` passes) and slot memory against
    private per-layer slots."""
    import numpy as np
    import torch

    from redundant_expert_balancing_amd.pool import MoEStack
    from redundant_expert_balancing_amd.synth import CONFIGS, make_dense, make_routing

    main = torch.cuda.current_stream()

    def time_passes(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(main)
            fn()
            b.record(main)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / n_layers)
        return round(float(np.median(ts)), 4)

    def build(cfg, nsets, backward):
        stack = MoEStack(cfg, n_layers, backward=backward, nsets=nsets)
        d = make_dense(cfg, "cuda", 0, which=("x", "W", "dy") if backward else ("x", "W"))
        ins = []
        for l in range(n_layers):
            r = make_routing(cfg, cfg.maxvio[l % len(cfg.maxvio)])
            stack.layers[l].w_all[:cfg.E].copy_(d["W"])
            ins.append((torch.from_numpy(r.topk_idx).cuda(), torch.from_numpy(r.gates).cuda()))
        del d["W"]
        return stack, d, ins

    out = {"layers": n_layers}
    cfg = CONFIGS["bench_shape"]
    stack, d, ins = build(cfg, 1, False)
    out["fwd_pool_bytes"] = stack.pool.nbytes
    out["fwd_private_slot_bytes"] = n_layers * cfg.R * cfg.B * cfg.H * cfg.Hp * 2

    def fwd():
        for l in range(n_layers):
            stack.forward_layer(l, ins[l][0], d["x"], ins[l][1])
    for mode in ("serial", "side_stream"):
        stack.overlap_forward = mode == "side_stream"
        out[f"fwd_{cfg.name}_{mode}_ms_per_layer"] = time_passes(fwd)
        print(f"[stack] {out}", file=sys.stderr, flush=True)
    assert all(layer.error_flags() == 0 for layer in stack.layers)
    stack.close()
    del stack, d, ins
    torch.cuda.empty_cache()

    cfg = CONFIGS["train_backward"]
    for nsets, overlap in ((1, False), (2, True)):
        stack, d, ins = build(cfg, nsets, True)
        stack.overlap_forward, stack.overlap_backward = False, overlap

        def bwd():
            for l in range(n_layers):
                stack.forward_layer(l, ins[l][0], d["x"], ins[l][1])
            torch.cuda.synchronize()
            return None

        # the backward alone is timed; each pass re-runs the forward untimed first
        ts = []
        for it in range(warmup + steps):
            bwd()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(main)
            for l in reversed(range(n_layers)):
                stack.backward_layer(l, d["dy"], ins[l][1])
            b.record(main)
            torch.cuda.synchronize()
            if it >= warmup:
                ts.append(a.elapsed_time(b) / n_layers)
        key = f"bwd_{cfg.name}_{nsets}set_{'side_stream' if overlap else 'serial'}"
        out[key + "_ms_per_layer"] = round(float(np.median(ts)), 4)
        out[key + "_pool_bytes"] = stack.pool.nbytes
        print(f"[stack] {out}", file=sys.stderr, flush=True)
        stack.close()
        del stack, d, ins
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def vendor_gemm(reps):
    """The grouped GEMM of the bench shape against the vendor library's dense GEMM
    of the same size, M = R*S*K slots by K = H by N = H' with one weight matrix
    (hipBLASLt through torch.mm, bf16 inputs, bf16 and float32 outputs), timed the
    same way in one process (caches flushed before every repetition). Measurement
    only: nothing on the path calls the vendor library."""
    import torch

    from redundant_expert_balancing_amd.layer import MoEProjection
    from redundant_expert_balancing_amd.synth import CONFIGS, make_dense, make_routing

    timed = _timer(reps)
    cfg = CONFIGS["bench_shape"]
    M, K, N = cfg.N * cfg.K, cfg.H, cfg.Hp
    flop = 2.0 * M * K * N

    def rate(us):
        tf = flop / (us * 1e-6) / 1e12
        return {"us": us, "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}

    out = {"shape": {"M": M, "K": K, "N": N}, "flop": flop}
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    w = (torch.randn((K, N), generator=g, device="cuda", dtype=torch.float32) / K ** 0.5).to(torch.bfloat16)
    c16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    out["hipblaslt_bf16_out"] = rate(timed(lambda: torch.mm(a, w, out=c16)))
    print(f"[vendor] bf16 out: {out['hipblaslt_bf16_out']}", file=sys.stderr, flush=True)
    del c16
    c32 = torch.mm(a, w, out_dtype=torch.float32)
    out["hipblaslt_fp32_out"] = rate(timed(lambda: torch.mm(a, w, out_dtype=torch.float32)))
    print(f"[vendor] fp32 out: {out['hipblaslt_fp32_out']}", file=sys.stderr, flush=True)
    del a, w, c32
    torch.cuda.empty_cache()

    d = make_dense(cfg, "cuda", 0, which=("x", "W"), w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEProjection(cfg, "cuda", w_all=d["W"])
    for target in cfg.maxvio:
        r = make_routing(cfg, target)
        topk = torch.from_numpy(r.topk_idx).cuda()
        layer.forward(topk, d["x"], torch.from_numpy(r.gates).cuda())
        out[f"grouped maxvio={r.maxvio:.3g}"] = rate(timed(layer.gemm_fwd))
        print(f"[vendor] grouped {target}: {out[f'grouped maxvio={r.maxvio:.3g}']}", file=sys.stderr,
              flush=True)
    print(json.dumps(out), flush=True)


def ffn_table(reps):
    """The full expert FFN on the balanced plan: forward stages at the bench shape
    for every imbalance point (plus the unfused gate/up GEMM + SwiGLU pass once),
    backward stages at the training-backward shape; TFLOP/s of every GEMM and
    GB/s of the SwiGLU passes."""
    import torch

    from redundant_expert_balancing_amd import _lib as L
    from redundant_expert_balancing_amd.ffn import MoEFFN
    from redundant_expert_balancing_amd.synth import CONFIGS, make_dense, make_routing

    timed = _timer(reps)
    out = {}

    def tf(flop, us):
        return round(flop / (us * 1e-6) / 1e12, 1)

    cfg = CONFIGS["bench_shape"]
    d = make_dense(cfg, "cuda", 0, which=("x", "W1", "W2"), w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEFFN(cfg, "cuda", w1_all=d["W1"], w2_all=d["W2"])
    slots = cfg.N * cfg.K
    f_up, f_down = 2.0 * slots * cfg.H * 2 * cfg.Hp, 2.0 * slots * cfg.Hp * cfg.H
    for i, target in enumerate(cfg.maxvio):
        r = make_routing(cfg, target)
        topk = torch.from_numpy(r.topk_idx).cuda()
        gates = torch.from_numpy(r.gates).cuda()
        layer.forward(topk, d["x"], gates)
        row = {"plan": timed(lambda: layer.plan(topk)),
               "prefetch_w1_w2": timed(layer.prefetch),
               "dispatch": timed(lambda: layer.dispatch(d["x"])),
               "gate_up_swiglu": timed(layer.gate_up),
               "down": timed(layer.down_proj),
               "combine": timed(lambda: layer.combine(gates))}
        row["gate_up_tflops"] = tf(f_up, row["gate_up_swiglu"])
        row["down_tflops"] = tf(f_down, row["down"])
        t = row["plan"] + row["dispatch"] + row["gate_up_swiglu"] + row["down"] + row["combine"]
        row["ffn_tokens_per_s"] = round(cfg.N / (t * 1e-6), 1)
        row["replicas"] = int((layer.replica_expert[:, :cfg.B] >= 0).sum())
        if i == 0:
            # the same projection unfused: GEMM to float32 h, then the SwiGLU pass
            h = torch.empty((slots, 2 * cfg.Hp), dtype=torch.float32, device="cuda")
            row["unfused_gemm"] = timed(lambda: L.moonep_grouped_gemm(
                layer.up, L.FWD, layer.xp, layer.w1_all, layer.cu_seqlens, h, None, None, layer.ws))
            row["unfused_swiglu"] = timed(lambda: L.moonep_swiglu(layer.shape, h, layer.act, None))
            sw_bytes = slots * (2 * cfg.Hp * 4 + cfg.Hp * 2)
            row["swiglu_gbs"] = round(sw_bytes / (row["unfused_swiglu"] * 1e-6) / 1e9, 1)
            del h
        out[f"fwd {cfg.name} maxvio={r.maxvio:.3g}"] = row
        print(f"[ffn] fwd {target}: {row}", file=sys.stderr, flush=True)
    del layer, d
    torch.cuda.empty_cache()

    cfg = CONFIGS["train_backward"]
    d = make_dense(cfg, "cuda", 0, which=("x", "W1", "W2", "dyH"), w_rows=cfg.E + cfg.R * cfg.B)
    layer = MoEFFN(cfg, "cuda", backward=True, w1_all=d["W1"], w2_all=d["W2"])
    slots = cfg.N * cfg.K
    f_up, f_down = 2.0 * slots * cfg.H * 2 * cfg.Hp, 2.0 * slots * cfg.Hp * cfg.H
    for target in cfg.maxvio:
        r = make_routing(cfg, target)
        topk = torch.from_numpy(r.topk_idx).cuda()
        gates = torch.from_numpy(r.gates).cuda()
        layer.forward(topk, d["x"], gates)
        layer.backward(d["dyH"], gates)
        up, dn, sh = layer.up, layer.down, layer.shape
        row = {"gate_up_swiglu": timed(layer.gate_up), "down": timed(layer.down_proj),
               "dispatch_dy": timed(lambda: L.moonep_dispatch(up, cfg.H, d["dyH"], layer.slot_map, gates, layer.dyp)),
               "dgrad_down": timed(lambda: L.moonep_grouped_gemm(dn, L.DGRAD, layer.dyp, layer.w2_all, layer.cu_seqlens, layer.da, None, None, layer.ws)),
               "wgrad_down": timed(lambda: L.moonep_grouped_gemm(dn, L.WGRAD, layer.act, layer.dyp, layer.cu_seqlens, None, layer.grad2, layer.red2, layer.ws)),
               "swiglu_backward": timed(lambda: L.moonep_swiglu_backward(sh, layer.hs, layer.da, layer.dh)),
               "dgrad_up": timed(lambda: L.moonep_grouped_gemm(up, L.DGRAD, layer.dh, layer.w1_all, layer.cu_seqlens, layer.dxp, None, None, layer.ws)),
               "wgrad_up": timed(lambda: L.moonep_grouped_gemm(up, L.WGRAD, layer.xp, layer.dh, layer.cu_seqlens, None, layer.grad1, layer.red1, layer.ws)),
               "unpermute": timed(lambda: L.moonep_combine(up, cfg.H, layer.dxp, layer.slot_map, None, layer.dx)),
               "reduce_grad_w1_w2": timed(lambda: (L.moonep_reduce_grad(up, layer.replica_expert, layer.red1, layer.grad1),
                                                    L.moonep_reduce_grad(dn, layer.replica_expert, layer.red2, layer.grad2)))}
        for k, f in (("gate_up_swiglu", f_up), ("down", f_down), ("dgrad_down", f_down),
                     ("wgrad_down", f_down), ("dgrad_up", f_up), ("wgrad_up", f_up)):
            row[k + "_tflops"] = tf(f, row[k])
        sb = slots * (2 * cfg.Hp * 2 + cfg.Hp * 4 + 2 * cfg.Hp * 2)
        row["swiglu_backward_gbs"] = round(sb / (row["swiglu_backward"] * 1e-6) / 1e9, 1)
        row["replicas"] = int((layer.replica_expert[:, :cfg.B] >= 0).sum())
        out[f"bwd {cfg.name} maxvio={r.maxvio:.3g}"] = row
        print(f"[ffn] bwd {target}: {row}", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
