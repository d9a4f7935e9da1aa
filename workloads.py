"""Seeded synthetic inputs for the MoE layer forward.

This module only draws random numbers and lays them out.  It holds none of
the layer's arithmetic (no routing, no softmax, no expert FFN), so both the
HIP path and the CPU oracle may take their inputs from here.

Workloads follow the layer shapes the pages work with:

* Qwen3-30B-A3B MoE block (the Qwen3-Omni issue "Training: Extremely Slow
  Deepspeed Engine initialization ...", concatenated experts
  ``gate_up_proj [E, H, 2I]`` and ``down_proj [E, I, H]``),
* one expert-parallel rank's received tokens in rank-major order
  (transformers PR "Qwen3 moe", ``Ep2DpParallel._token_dispatch``),

with Gaussian values, since no trained weights or datasets are available.

Draw order (one ``torch.Generator`` per workload, seeded):
router weight, gate_up, down, then hidden states (for the EP-rank workload,
the hidden states of source ranks 0..R-1 in order).  Every draw is a standard
normal scaled by its std in float32; bf16 workloads then round to bfloat16
(round-to-nearest-even, torch's ``.to(torch.bfloat16)``).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

__all__ = ["Workload", "EPWorkload", "CONFIGS", "make", "make_layer",
           "make_ep_rank", "zipf_router_bias", "integer_grid_layer",
           "shared_expert_weights"]


@dataclasses.dataclass
class Workload:
    """Inputs of one token-choice MoE layer forward (all CPU tensors)."""
    name: str
    T: int
    H: int
    I: int
    E: int
    top_k: int
    norm_topk_prob: bool
    dtype: torch.dtype
    hidden_states: torch.Tensor      # [T, H]   dtype
    router_weight: torch.Tensor      # [E, H]   dtype (nn.Linear(H, E) layout)
    router_bias: Optional[torch.Tensor]  # [E] float32 or None
    gate_up: torch.Tensor            # [E, H, 2I] dtype, gate = cols [0, I)
    down: torch.Tensor               # [E, I, H] dtype

    @property
    def N(self) -> int:
        return self.T * self.top_k


@dataclasses.dataclass
class EPWorkload:
    """One expert-parallel rank's share: its local experts and the hidden
    states of every source rank (routing them is the method's job)."""
    name: str
    R: int                 # number of source ranks
    T_per_rank: int
    H: int
    I: int
    E: int                 # global experts
    E_local: int
    local_lo: int          # first local expert id (contiguous block)
    top_k: int
    norm_topk_prob: bool
    dtype: torch.dtype
    router_weight: torch.Tensor      # [E, H]
    gate_up: torch.Tensor            # [E_local, H, 2I]
    down: torch.Tensor               # [E_local, I, H]
    source_hidden: list              # R tensors [T_per_rank, H]


def _normal(g: torch.Generator, shape, std: float, dtype: torch.dtype) -> torch.Tensor:
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype) if dtype != torch.float32 else t


def zipf_router_bias(E: int, s: float = 1.2) -> torch.Tensor:
    """Per-expert logit bias ``b_e = -s * ln(1 + e)``: the log of the
    unnormalised Zipf(s) mass of rank ``e + 1``.  Added to the router logits
    it skews expert popularity toward low ids."""
    return torch.tensor([-s * math.log(1.0 + e) for e in range(E)], dtype=torch.float32)


def make_layer(name: str, T: int, H: int, I: int, E: int, top_k: int,
               norm_topk_prob: bool = True, dtype: torch.dtype = torch.bfloat16,
               seed: int = 0, weight_std: float = 0.02, x_std: float = 1.0,
               router_bias: Optional[torch.Tensor] = None) -> Workload:
    g = torch.Generator().manual_seed(seed)
    wr = _normal(g, (E, H), weight_std, dtype)
    gu = _normal(g, (E, H, 2 * I), weight_std, dtype)
    dn = _normal(g, (E, I, H), weight_std, dtype)
    x = _normal(g, (T, H), x_std, dtype)
    return Workload(name, T, H, I, E, top_k, norm_topk_prob, dtype, x, wr,
                    router_bias, gu, dn)


def shared_expert_weights(H: int, Is: int, dtype: torch.dtype = torch.bfloat16, seed: int = 0,
                          weight_std: float = 0.02):
    """Weights of a shared expert (the MindSpore moe.py page's FeedForward)
    as nn.Linear stores them: w1 [Is, H], w2 [H, Is], w3 [Is, H], drawn in
    that order from their own generator (seed + 1000, so they never repeat a
    layer's draws)."""
    g = torch.Generator().manual_seed(seed + 1000)
    w1 = _normal(g, (Is, H), weight_std, dtype)
    w2 = _normal(g, (H, Is), weight_std, dtype)
    w3 = _normal(g, (Is, H), weight_std, dtype)
    return w1, w2, w3


def make_ep_rank(name: str = "ep_rank_235b", R: int = 8, T_per_rank: int = 4096,
                 H: int = 4096, I: int = 1536, E: int = 128, E_local: int = 16,
                 rank: int = 0, top_k: int = 8, norm_topk_prob: bool = True,
                 dtype: torch.dtype = torch.bfloat16, seed: int = 0,
                 weight_std: float = 0.02) -> EPWorkload:
    g = torch.Generator().manual_seed(seed)
    wr = _normal(g, (E, H), weight_std, dtype)
    gu = _normal(g, (E_local, H, 2 * I), weight_std, dtype)
    dn = _normal(g, (E_local, I, H), weight_std, dtype)
    xs = [_normal(g, (T_per_rank, H), 1.0, dtype) for _ in range(R)]
    return EPWorkload(name, R, T_per_rank, H, I, E, E_local, rank * E_local,
                      top_k, norm_topk_prob, dtype, wr, gu, dn, xs)


def integer_grid_layer(T: int, H: int, I: int, E: int, top_k: int,
                       norm_topk_prob: bool = True, dtype=torch.bfloat16,
                       seed: int = 0, levels: int = 2) -> Workload:
    """Inputs whose router logits are exact in float32 under any summation
    order: x in {-levels..levels}/8 and router weights in
    {-levels..levels}/16, so every product is a multiple of 2^-7 and every
    partial sum stays far inside float32's 24-bit significand.  Exact logit
    ties between experts are frequent, which exercises the tie rule."""
    g = torch.Generator().manual_seed(seed)
    wr = torch.randint(-levels, levels + 1, (E, H), generator=g).float() / 16.0
    gu = _normal(g, (E, H, 2 * I), 0.02, torch.float32)
    dn = _normal(g, (E, I, H), 0.02, torch.float32)
    x = torch.randint(-levels, levels + 1, (T, H), generator=g).float() / 8.0
    cast = (lambda t: t.to(dtype)) if dtype != torch.float32 else (lambda t: t)
    return Workload("integer_grid", T, H, I, E, top_k, norm_topk_prob, dtype,
                    cast(x), cast(wr), None, cast(gu), cast(dn))


# The five named workloads.  Sizes and distributions follow the layer shapes
# above; seed 0 for all.
CONFIGS: Dict[str, dict] = {
    "tiny_fp32": dict(kind="layer", T=64, H=128, I=64, E=8, top_k=2,
                      norm_topk_prob=True, dtype=torch.float32),
    "qwen3_30b_a3b_prefill": dict(kind="layer", T=4096, H=2048, I=768, E=128,
                                  top_k=8, norm_topk_prob=True, dtype=torch.bfloat16),
    "qwen3_30b_a3b_decode": dict(kind="layer", T=64, H=2048, I=768, E=128,
                                 top_k=8, norm_topk_prob=True, dtype=torch.bfloat16),
    "ep_rank_235b": dict(kind="ep", R=8, T_per_rank=4096, H=4096, I=1536, E=128,
                         E_local=16, top_k=8, norm_topk_prob=True,
                         dtype=torch.bfloat16),
    "qwen3_30b_a3b_skewed": dict(kind="layer", T=16384, H=2048, I=768, E=128,
                                 top_k=8, norm_topk_prob=True, dtype=torch.bfloat16,
                                 zipf_s=1.2),
}


def make(name: str, seed: int = 0, **overrides):
    """Build a named workload (optionally with some sizes overridden, e.g. a
    smaller T for a quick case)."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    if kind == "ep":
        return make_ep_rank(name=name, seed=seed, **cfg)
    zipf_s = cfg.pop("zipf_s", None)
    bias = zipf_router_bias(cfg["E"], zipf_s) if zipf_s is not None else None
    return make_layer(name=name, seed=seed, router_bias=bias, **cfg)


def random_topk_ids(T: int, E: int, k: int, seed: int = 0,
                    popularity: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Random expert selections: for each token, k distinct experts drawn
    without replacement (uniformly, or in proportion to ``popularity``).
    A stand-in for a router's output when only the permutation is tested."""
    g = torch.Generator().manual_seed(seed)
    p = torch.ones(E) if popularity is None else popularity.float()
    p = p.expand(T, E).contiguous()
    return torch.multinomial(p, k, replacement=False, generator=g).to(torch.int32)
