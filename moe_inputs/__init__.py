"""Seeded synthetic inputs for the one-GPU MoE layer.

This module only draws random tensors with the shapes, scales and structure of
the workloads below; it holds none of the layer's arithmetic.  Both sides
of a parity check (the HIP library and the CPU oracle) are fed from here.

Seeding: every tensor, and every expert's slice of a weight tensor, gets its
own child seed derived with ``numpy.random.SeedSequence(base_seed,
spawn_key=(tensor_id, expert))``; that 64-bit value seeds a
``torch.Generator`` on the device where the tensor is drawn.  Any expert can
therefore be regenerated on its own.  Draws are N(0,1) in fp32, scaled by the
stated standard deviation in fp32, then rounded once (round-to-nearest-even)
to bf16 for the bf16 workloads.  The same seed gives the same values on the
same device type; CPU and GPU draws differ, so a test draws once and hands the
same tensors to both sides.

Weight layouts are the ones the C ABI takes ([out_features, in_features] per
expert, i.e. the contraction dimension contiguous):
    w_router [E, d]      router scores  l = x . w_router^T (+ router_bias)
    w_gate   [E, F, d]   g = x . w_gate[e]^T
    w_up     [E, F, d]   u = x . w_up[e]^T
    w_down   [E, d, F]   y = h . w_down[e]^T
    ws_gate, ws_up [Fs, d]; ws_down [d, Fs]   the shared expert
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1
DTYPE_F32 = 0
DTYPE_BF16 = 1

# Stable ids for the child seeds; never renumber.
_TENSOR_IDS = {
    "x": 1, "w_router": 2, "router_bias": 3, "score_bias": 4,
    "w_gate": 5, "w_up": 6, "w_down": 7,
    "ws_gate": 8, "ws_up": 9, "ws_down": 10, "dy": 11, "zipf_rank": 12,
    "logits": 13, "routing": 14, "gates": 15, "rows": 16,
}


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One workload: the layer's parameters plus the recipe of its inputs."""
    name: str
    T: int                      # tokens
    d: int                      # hidden size
    E: int                      # routed experts
    k: int                      # experts per token
    F: int                      # routed expert FFN width
    F_shared: int = 0           # width of the shared expert (every token), 0 = none
    n_groups: int = 1           # expert groups for group-limited routing
    topk_groups: int = 1        # groups kept per token
    score: int = SCORE_SOFTMAX
    renorm: int = 1             # renormalise the k gates over the selected set
    dtype: int = DTYPE_BF16
    wgrad_dtype: int = DTYPE_F32    # storage of the weight gradients
    wgrad_mx: int = 0               # MXFP8 backward: weight gradients in MXFP8 too
    x_std: float = 1.0
    w_std: float = 0.02
    router_std: float = 0.02
    score_bias_std: float = 0.0     # per-expert selection bias (sigmoid scoring)
    zipf_s: float = 0.0             # per-expert router offsets -s*ln(rank)
    backward: bool = False          # the workload includes the backward pass
    seed: int = 0

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == DTYPE_F32 else torch.bfloat16

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    def expert_params(self) -> int:
        """Parameters of one routed expert (three matrices)."""
        return 3 * self.d * self.F


# The workloads, named by what they are.
CONFIGS: Dict[str, MoEConfig] = {
    # Tiny fp32 forward: top-2 of 8, renormalised softmax gates.
    "tiny_fp32": MoEConfig("tiny_fp32", T=256, d=128, E=8, k=2, F=256,
                           dtype=DTYPE_F32, router_std=0.02),
    # Mixtral-shape bf16 forward; near-uniform router logits (std ~0.064).
    "mixtral_t4096": MoEConfig("mixtral_t4096", T=4096, d=4096, E=8, k=2,
                               F=14336, router_std=1e-3),
    # DeepSeek-V3-shape bf16 forward: sigmoid scores, per-expert selection
    # bias, 8 groups keep 4, top-8 of 256, plus one shared expert.
    "deepseek_v3_t8192": MoEConfig("deepseek_v3_t8192", T=8192, d=7168,
                                   E=256, k=8, F=2048, F_shared=2048,
                                   n_groups=8, topk_groups=4,
                                   score=SCORE_SIGMOID, score_bias_std=0.1),
    # Qwen3-30B-A3B-shape bf16 forward with Zipf(1.2) router offsets: skewed
    # loads, some experts get no tokens.
    "qwen3_30b_skewed_t16384": MoEConfig("qwen3_30b_skewed_t16384", T=16384,
                                         d=2048, E=128, k=8, F=768,
                                         zipf_s=1.2),
    # One rank's share of the DeepSeek-V3 shape under 8-way expert
    # parallelism: 32 local experts receiving about T*k = 65,536 rows (2,048
    # per expert).  Routing is drawn locally (top-8 of the 32 experts) so the
    # grouped FFN sees that row count; it stands in for the rows a dispatch
    # would deliver from the other ranks (the shared expert stays with the
    # token's own rank and is left out).
    "deepseek_v3_ep8_rank_t8192": MoEConfig("deepseek_v3_ep8_rank_t8192", T=8192,
                                            d=7168, E=32, k=8, F=2048),
    # DeepSeek-V3-shape bf16 training step: the forward workload above plus
    # the backward of the sigmoid group-limited router and the shared expert.
    "deepseek_v3_train_t8192": MoEConfig("deepseek_v3_train_t8192", T=8192,
                                         d=7168, E=256, k=8, F=2048,
                                         F_shared=2048, n_groups=8,
                                         topk_groups=4, score=SCORE_SIGMOID,
                                         score_bias_std=0.1, backward=True),
    # Qwen3-235B-A22B-shape bf16 training step (forward + backward).
    "qwen3_235b_train_t8192": MoEConfig("qwen3_235b_train_t8192", T=8192,
                                        d=4096, E=128, k=8, F=1536,
                                        backward=True),
}


def child_seed(base_seed: int, tensor: str, expert: int = -1) -> int:
    key = (_TENSOR_IDS[tensor], expert + 1)
    ss = np.random.SeedSequence(entropy=base_seed, spawn_key=key)
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std, dtype, device, seed):
    """N(0, std^2) drawn in fp32, scaled in fp32, rounded once to ``dtype``."""
    t = torch.randn(shape, generator=_gen(device, seed), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def expert_weight(cfg: MoEConfig, name: str, e: int, device="cpu"):
    """One expert's slice of w_gate / w_up ([F, d]) or w_down ([d, F])."""
    shape = (cfg.d, cfg.F) if name == "w_down" else (cfg.F, cfg.d)
    return normal(shape, cfg.w_std, cfg.torch_dtype, device,
                  child_seed(cfg.seed, name, e))


def make_inputs(cfg: MoEConfig, device="cpu", with_weights=True) -> dict:
    """All inputs of one workload, drawn on ``device``."""
    dt = cfg.torch_dtype
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = normal((cfg.T, cfg.d), cfg.x_std, dt, device,
                      child_seed(cfg.seed, "x"))
    out["w_router"] = normal((cfg.E, cfg.d), cfg.router_std, dt, device,
                             child_seed(cfg.seed, "w_router"))
    out["router_bias"] = None
    if cfg.zipf_s > 0:
        # Per-expert offsets -s*ln(rank), ranks a seeded permutation of 1..E.
        rng = np.random.Generator(np.random.PCG64(
            child_seed(cfg.seed, "zipf_rank")))
        ranks = rng.permutation(cfg.E) + 1
        off = np.array([-cfg.zipf_s * math.log(r) for r in ranks],
                       dtype=np.float32)
        out["router_bias"] = torch.from_numpy(off).to(device)
    out["score_bias"] = None
    if cfg.score_bias_std > 0:
        out["score_bias"] = normal((cfg.E,), cfg.score_bias_std,
                                   torch.float32, device,
                                   child_seed(cfg.seed, "score_bias"))
    if with_weights:
        for name in ("w_gate", "w_up", "w_down"):
            shape = ((cfg.E, cfg.d, cfg.F) if name == "w_down"
                     else (cfg.E, cfg.F, cfg.d))
            w = torch.empty(shape, dtype=dt, device=device)
            for e in range(cfg.E):
                w[e].copy_(expert_weight(cfg, name, e, device))
            out[name] = w
        for name in ("ws_gate", "ws_up", "ws_down"):
            out[name] = None
        if cfg.F_shared > 0:
            fs = cfg.F_shared
            out["ws_gate"] = normal((fs, cfg.d), cfg.w_std, dt, device,
                                    child_seed(cfg.seed, "ws_gate"))
            out["ws_up"] = normal((fs, cfg.d), cfg.w_std, dt, device,
                                  child_seed(cfg.seed, "ws_up"))
            out["ws_down"] = normal((cfg.d, fs), cfg.w_std, dt, device,
                                    child_seed(cfg.seed, "ws_down"))
    out["dy"] = None
    if cfg.backward:
        out["dy"] = normal((cfg.T, cfg.d), 1.0, dt, device,
                           child_seed(cfg.seed, "dy"))
    return out


def round_robin_topk(T: int, E: int, k: int) -> torch.Tensor:
    """Deliberately balanced routing: token t picks experts (t*k + j) mod E.

    The k picks of a token are distinct when k <= E.
    """
    t = torch.arange(T, dtype=torch.int64).unsqueeze(1)
    j = torch.arange(k, dtype=torch.int64).unsqueeze(0)
    return ((t * k + j) % E).to(torch.int32)


def weighted_round_robin_topk(T: int, E: int, k: int, weights) -> torch.Tensor:
    """Deliberately imbalanced round-robin routing: a cyclic schedule lists,
    in round r = 0, 1, ..., every expert e with weights[e] > r in ascending
    order; token t takes the k entries of the schedule from position t*k on
    (cyclically).  Expert e then appears weights[e] times per cycle, so its
    row count is weights[e] * T*k / len(schedule) when the cycle divides
    T*k; experts of weight 0 get no rows.  Raises when some window of k
    consecutive entries repeats an expert (the k picks must be distinct)."""
    w = [int(v) for v in weights]
    assert len(w) == E and min(w) >= 0
    sched = [e for r in range(max(w)) for e in range(E) if w[e] > r]
    L = len(sched)
    for p in range(L):
        win = [sched[(p + j) % L] for j in range(k)]
        if len(set(win)) != k:
            raise ValueError("the weighted schedule repeats an expert within k entries")
    pos = (torch.arange(T, dtype=torch.int64).unsqueeze(1) * k +
           torch.arange(k, dtype=torch.int64).unsqueeze(0)) % L
    return torch.as_tensor(sched, dtype=torch.int32)[pos]


def planted_logits(topk_idx: torch.Tensor, E: int, seed: int) -> torch.Tensor:
    """fp32 router scores whose k best entries per token are topk_idx, in
    that order: background N(0, 0.1^2), pick j set to 8 - j/2."""
    T, k = topk_idx.shape
    t = normal((T, E), 0.1, torch.float32, "cpu", child_seed(seed, "logits"))
    vals = 8.0 - 0.5 * torch.arange(k, dtype=torch.float32)
    t.scatter_(1, topk_idx.long(), vals.expand(T, k).contiguous())
    return t


def random_topk(T: int, E: int, k: int, seed: int, weights=None) -> torch.Tensor:
    """T rows of k distinct experts in [0, E), drawn without replacement with
    per-expert selection weights (uniform when None; a skewed vector leaves
    some experts without rows)."""
    rng = np.random.Generator(np.random.PCG64(child_seed(seed, "routing")))
    p = None
    if weights is not None:
        p = np.asarray(weights, dtype=np.float64)
        p = p / p.sum()
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        out[t] = rng.choice(E, size=k, replace=False, p=p)
    return torch.from_numpy(out)


def random_gates(T: int, k: int, seed: int) -> torch.Tensor:
    """Positive fp32 combine weights (not normalised)."""
    rng = np.random.Generator(np.random.PCG64(child_seed(seed, "gates")))
    return torch.from_numpy(rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32))


def random_logits(T: int, E: int, seed: int, std: float = 1.0,
                  quantum: float = 0.0) -> torch.Tensor:
    """fp32 router scores; with quantum > 0 they are rounded to multiples of
    it, which plants exact ties."""
    t = normal((T, E), std, torch.float32, "cpu", child_seed(seed, "logits"))
    if quantum > 0:
        t = torch.round(t / quantum) * quantum
    return t
