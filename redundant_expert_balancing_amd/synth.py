"""Seeded synthetic inputs: a simulated router and the dense tensors of one MoE layer.

This module is the only code that the GPU path and the CPU oracle share. It holds
no arithmetic of the balancing method itself: it plays the part of the training
framework that sits above the library (the router that picks each token's top-K
experts, and the activations / weights / upstream gradients), producing inputs
that both sides consume unchanged.

Workload recipe (the pages benchmark on synthetic routing drawn from one shared
seed at several imbalance levels -- ai-maestro.online "Moonshot AI open-sources
MoonEP", section "Benchmarks against DeepEP v2"):

* ``numpy.random.SeedSequence(seed).spawn(5)`` gives five PCG64 streams, used for
  (router logits, expert bias profile, x, W, dy).
* logits ~ N(0, 1) in float32, shape [R*S, E]; score = logits + alpha * z
  (float32), where z is the per-expert bias profile: N(0, 1) by default, or the
  fixed "overflow" profile that makes one rank ask for more distinct remote
  experts than an inference-mode prefetch budget holds.
* top-K by score descending, ties to the lower expert id; k order is score
  descending. Gates are the softmax over the K selected scores (float64, stored
  float32).
* alpha is bisected so the routing's imbalance max_e(T_e / Tbar) - 1 hits the
  target; the results are tabulated in ``ALPHA`` (re-derive with
  ``python -m redundant_expert_balancing_amd.synth``).
* x ~ N(0, 1), W ~ N(0, 1/H), dy ~ N(0, 1), rounded once to the layer dtype
  (round-to-nearest-even for bfloat16). Dense tensors are drawn with torch's
  generator on the device that will hold them, seeded from the same spawned
  streams, so large layers never pass through host memory.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = ["LayerConfig", "CONFIGS", "ALPHA", "Routing", "make_routing",
           "routing_imbalance", "calibrate_alpha", "make_dense", "stream_seed"]


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape of one MoE layer spread over R expert-parallel ranks."""
    name: str
    R: int        # expert-parallel ranks (virtual: partitions of one GPU)
    S: int        # tokens per rank
    E: int        # routed experts
    K: int        # experts per token
    B: int        # prefetch (replica) slots per rank
    H: int        # hidden size
    Hp: int       # expert intermediate size H'
    dtype: str    # "bf16" or "fp32"
    mode: str     # "train" or "infer"
    maxvio: tuple  # imbalance targets swept for this layer
    profile: str = "gauss"
    backward: bool = False

    @property
    def G(self) -> int:
        return self.E // self.R

    @property
    def N(self) -> int:
        return self.R * self.S

    @property
    def SK(self) -> int:
        return self.S * self.K


CONFIGS = {
    c.name: c for c in [
        LayerConfig("tiny_fp32_train", 4, 64, 16, 2, 4, 128, 64, "fp32", "train", (1.0,)),
        LayerConfig("bf16_train_mild", 8, 1024, 64, 4, 8, 1024, 512, "bf16", "train", (0.2,)),
        LayerConfig("bench_shape", 8, 8192, 384, 8, 48, 7168, 2048, "bf16", "train",
                    (0.2, 1.0, 10.0, 20.0)),
        LayerConfig("infer_overflow", 16, 4096, 256, 8, 4, 4096, 1536, "bf16", "infer",
                    (10.0,), profile="overflow"),
        # maxvio 20 is out of reach here: a token names an expert at most once, so
        # T_e <= R*S and max maxvio = E/K - 1 = 15. The sweep point is clamped to 15.
        LayerConfig("train_backward", 8, 4096, 128, 8, 16, 4096, 1408, "bf16", "train",
                    (15.0,), backward=True),
    ]
}

# alpha per (config name, maxvio target), seed 0, from calibrate_alpha().
ALPHA = {
    ("tiny_fp32_train", 1.0): 0.49609375,  # maxvio 1.000000
    ("bf16_train_mild", 0.2): 0.0361328125,  # maxvio 0.199219
    ("bench_shape", 0.2): 0.029296875,  # maxvio 0.199707
    ("bench_shape", 1.0): 0.111175537109375,  # maxvio 1.000244
    ("bench_shape", 10.0): 0.544921875,  # maxvio 10.000244
    ("bench_shape", 20.0): 0.8795346021652222,  # maxvio 20.000000
    ("infer_overflow", 10.0): 1.4960365295410156,  # maxvio 10.000000
    ("train_backward", 15.0): 9.985006809292827,  # maxvio 15.000000
}


def stream_seed(seed: int, which: int) -> int:
    """A 63-bit integer seed for stream ``which`` (0 logits, 1 profile, 2 x, 3 W, 4 dy;
    for the full expert FFN 5 W1, 6 W2, 7 dy of width H). Child i of a SeedSequence
    does not depend on how many children are spawned, so streams 0-4 are unchanged
    by the later ones."""
    ss = np.random.SeedSequence(seed).spawn(8)[which]
    return int(ss.generate_state(2, dtype=np.uint64)[0] >> np.uint64(1))


def _rng(seed: int, which: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(5)[which]))


_CHUNK = 2048   # router rows per block: keeps every temporary cache-sized


def _profile(cfg: LayerConfig, seed: int) -> np.ndarray:
    if cfg.profile == "gauss":
        return _rng(seed, 1).standard_normal(cfg.E).astype(np.float32)
    if cfg.profile == "overflow":
        # Group 0 mildly hot, the first expert of group 1 very hot, group 2 cold:
        # rank 2 then borrows from a hot group whose load is spread over many
        # experts, so it needs more distinct remote experts than B slots.
        G = cfg.G
        z = np.zeros(cfg.E, dtype=np.float32)
        z[0:G] = 0.3
        z[G] = 1.0
        z[2 * G:3 * G] = -2.0
        return z
    raise ValueError(f"unknown profile {cfg.profile!r}")


def _topk_rows(s: np.ndarray, K: int) -> np.ndarray:
    """Ids of the K largest entries per row, ties to the lower id, score-descending."""
    E = s.shape[1]
    kth = np.partition(s, E - K, axis=1)[:, E - K:E - K + 1]   # K-th largest value
    take = s >= kth
    for r in np.nonzero(take.sum(axis=1) > K)[0]:   # ties at the cut: keep lower ids
        above = np.nonzero(s[r] > kth[r, 0])[0]
        tied = np.nonzero(s[r] == kth[r, 0])[0][:K - len(above)]
        take[r] = False
        take[r, above] = True
        take[r, tied] = True
    ids = np.nonzero(take)[1].reshape(-1, K)                    # ascending id per row
    vals = np.take_along_axis(s, ids, axis=1)
    order = np.argsort(-vals, axis=1, kind="stable")            # score desc, id asc
    return np.take_along_axis(ids, order, axis=1)


def _route(cfg: LayerConfig, seed: int, alpha: float, with_gates: bool = True):
    """Top-K ids (and gates) of score = logits + alpha*z, streamed in row blocks.

    The logits come from one PCG64 stream drawn block after block, which yields
    the same values as drawing the whole [R*S, E] matrix at once.
    """
    rng = _rng(seed, 0)
    az = _profile(cfg, seed) * np.float32(alpha)
    topk = np.empty((cfg.N, cfg.K), dtype=np.int32)
    gates = np.empty((cfg.N, cfg.K), dtype=np.float32) if with_gates else None
    for r0 in range(0, cfg.N, _CHUNK):
        n = min(_CHUNK, cfg.N - r0)
        score = rng.standard_normal((n, cfg.E), dtype=np.float32)
        score += az
        ids = _topk_rows(score, cfg.K)
        topk[r0:r0 + n] = ids
        if with_gates:
            sel = np.take_along_axis(score, ids, axis=1).astype(np.float64)
            ex = np.exp(sel - sel.max(axis=1, keepdims=True))
            gates[r0:r0 + n] = ex / ex.sum(axis=1, keepdims=True)
    return topk, gates


def _expert_counts(topk: np.ndarray, E: int) -> np.ndarray:
    return np.bincount(topk.reshape(-1), minlength=E)


def routing_imbalance(topk: np.ndarray, cfg: LayerConfig) -> float:
    """max_e(T_e / Tbar) - 1 with Tbar = R*S*K/E, used only to steer alpha."""
    T = _expert_counts(topk, cfg.E)
    return float(T.max()) / (cfg.N * cfg.K / cfg.E) - 1.0


@dataclasses.dataclass
class Routing:
    cfg: LayerConfig
    alpha: float
    topk_idx: np.ndarray   # int32 [R*S, K]
    gates: np.ndarray      # float32 [R*S, K]
    maxvio: float


def make_routing(cfg: LayerConfig, target: float, seed: int = 0,
                 alpha: float | None = None) -> Routing:
    """Router output for ``cfg`` at imbalance ``target`` (alpha from ``ALPHA`` if known)."""
    if alpha is None:
        alpha = ALPHA.get((cfg.name, float(target)))
        if alpha is None:
            alpha = calibrate_alpha(cfg, target, seed)
    topk, gates = _route(cfg, seed, alpha)
    return Routing(cfg, float(alpha), topk, gates, routing_imbalance(topk, cfg))


def calibrate_alpha(cfg: LayerConfig, target: float, seed: int = 0, steps: int = 40) -> float:
    """Bisect alpha in [0, 64] for the target imbalance; keep the closest alpha seen.

    For a target at the ceiling E/K - 1, return the smallest alpha that reaches it.
    """
    ceiling = cfg.E / cfg.K - 1.0
    lo, hi = 0.0, 64.0
    best, best_err = 0.0, float("inf")
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        mv = routing_imbalance(_route(cfg, seed, mid, with_gates=False)[0], cfg)
        if target >= ceiling:
            if mv >= target - 1e-12:
                best, hi = mid, mid
            else:
                lo = mid
            continue
        if abs(mv - target) < best_err:
            best, best_err = mid, abs(mv - target)
        if mv < target:
            lo = mid
        else:
            hi = mid
    return best


def make_dense(cfg: LayerConfig, device="cpu", seed: int = 0, which=("x", "W", "dy"),
               w_rows: int | None = None):
    """Layer tensors in the layer dtype, drawn on ``device``:

      x [R*S,H] ~ N(0,1);  W [w_rows,H,H'] ~ N(0,1/H);  dy [R*S,H'] ~ N(0,1)
      full expert FFN:  W1 [w_rows,H,2H'] ~ N(0,1/H) (gate/up),
                        W2 [w_rows,H',H] ~ N(0,1/H') (down),  dyH [R*S,H] ~ N(0,1)

    Only the first E rows of a weight are drawn (the home experts); ``w_rows``
    (default E) may reserve further rows, left uninitialised, for the prefetch slots.
    """
    import torch
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    weights = {"W": (3, cfg.H, cfg.Hp, cfg.H), "W1": (5, cfg.H, 2 * cfg.Hp, cfg.H),
               "W2": (6, cfg.Hp, cfg.H, cfg.Hp)}
    rows_of = {"x": (2, cfg.H), "dy": (4, cfg.Hp), "dyH": (7, cfg.H)}
    out = {}
    for name in which:
        g = torch.Generator(device=device)
        if name in weights:
            stream, d0, d1, fan_in = weights[name]
            g.manual_seed(stream_seed(seed, stream))
            rows = cfg.E if w_rows is None else w_rows
            t = torch.empty((rows, d0, d1), dtype=dt, device=device)
            buf = torch.empty((d0, d1), dtype=torch.float32, device=device)
            for e in range(cfg.E):      # expert by expert: fp32 staging stays small
                buf.normal_(0.0, fan_in ** -0.5, generator=g)
                t[e].copy_(buf)
        elif name in rows_of:
            stream, width = rows_of[name]
            g.manual_seed(stream_seed(seed, stream))
            buf = torch.empty((cfg.N, width), dtype=torch.float32, device=device)
            buf.normal_(0.0, 1.0, generator=g)
            t = buf.to(dt)
        else:
            raise ValueError(name)
        out[name] = t
    return out


if __name__ == "__main__":
    for (name, target) in ALPHA:
        cfg = CONFIGS[name]
        a = calibrate_alpha(cfg, target)
        r = make_routing(cfg, target, alpha=a)
        print(f'    ("{name}", {target}): {a!r},  # maxvio {r.maxvio:.6f}')
