"""Seeded synthetic workloads for MoE top-k routing, dispatch and combine.

This module only draws random inputs; it computes nothing that routing,
dispatch or combine compute.  Both the CPU oracle tests and the GPU path take
their inputs from here, so the two sides always see identical bytes.

Shapes follow the model shapes the pages discuss: the Mixtral special case of
routing ("Lower latency and higher throughput with multi-node DeepSeek
deployment", section "MoE Router"), DeepSeek-V3 with 256 routed experts and 8
experts per token (same page, "Expert parallelism"), and Kimi-K2 / DeepSeek-V3
at hidden size 7168 ("Enabling trillion-parameter models on AWS EFA",
section "Evaluation").  Model names here are shapes only; no weights or
datasets are involved.

Recipe (per config, one integer seed, default 0):

* ``numpy.random.SeedSequence(seed).spawn(4)`` gives independent PCG64
  streams for logits, token activations ``x``, expert outputs ``y`` and the
  expert-popularity permutation.
* logits: ``standard_normal((T, E), float32)``.
* Zipf(s) popularity (decode / imbalanced configs): expert ``e`` gets rank
  ``r = perm[e] + 1`` and ``float32(log(r**-s / sum_r' r'**-s))`` is added
  to its logit column.
* hot expert (imbalanced config): the expert whose Zipf rank is
  ``hot_rank`` gets ``+hot_bias`` added to its logit column.
* ``x`` and ``y``: ``standard_normal(float32)`` rounded to bf16 by torch's CPU
  conversion; returned as raw uint16 bit patterns.
* ``y`` has ``T*k`` rows, i.e. one expert-output row per dispatched row.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Config", "CONFIGS", "Workload", "make", "bf16_from_f32", "seed_streams"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int            # tokens
    H: int            # hidden size (bf16 elements per row)
    E: int            # routed experts
    k: int            # experts per token
    R: int            # virtual ranks; E // R local experts per rank
    zipf_s: Optional[float] = None
    hot_bias: Optional[float] = None
    hot_rank: Optional[int] = None
    note: str = ""

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def L(self) -> int:
        return self.E // self.R


CONFIGS = {
    c.name: c
    for c in [
        Config("tiny", T=16, H=256, E=8, k=2, R=1,
               note="small case; the oracle finishes in well under a second"),
        Config("mixtral", T=4096, H=4096, E=8, k=2, R=8,
               note="Mixtral-8x7B shape, 8 virtual ranks x 1 local expert"),
        Config("dsv3_decode", T=128, H=7168, E=256, k=8, R=32, zipf_s=1.0,
               note="DeepSeek-V3 decode share of EP32, Zipf(1.0) skew"),
        Config("dsv3_prefill", T=8192, H=7168, E=256, k=8, R=32,
               note="DeepSeek-V3 prefill share of EP32, near-uniform load"),
        Config("kimi_k2", T=4096, H=7168, E=384, k=8, R=48, zipf_s=1.2,
               hot_bias=4.0, hot_rank=250,
               note="Kimi-K2 shape, EP48 share, Zipf(1.2) plus one hot expert"),
    ]
}


def seed_streams(seed: int, n: int = 4):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 samples to bf16 with torch's CPU conversion; uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@dataclasses.dataclass
class Workload:
    cfg: Config
    seed: int
    logits: np.ndarray          # float32 [T, E]
    x: np.ndarray               # uint16 (bf16 bits) [T, H]
    y: Optional[np.ndarray]     # uint16 (bf16 bits) [T*k, H], or None
    expert_rank: np.ndarray     # int64 [E]: Zipf rank of each expert (1 = most popular)
    hot_expert: Optional[int]


def zipf_log_popularity(E: int, s: float) -> np.ndarray:
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    return np.log(p / p.sum())


def make(cfg: Config | str, seed: int = 0, *, with_y: bool = True,
         T: Optional[int] = None) -> Workload:
    """Build the seeded inputs of ``cfg``.

    ``T`` overrides the token count (a prefix sample of the same distribution:
    rows are drawn in order, so ``make(cfg, T=n).logits`` equals the first
    ``n`` rows of the full workload's logits).
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    T = cfg.T if T is None else int(T)
    g_logits, g_x, g_y, g_perm = seed_streams(seed, 4)

    logits = g_logits.standard_normal((T, cfg.E), dtype=np.float32)
    perm = g_perm.permutation(cfg.E)
    expert_rank = perm.astype(np.int64) + 1
    hot = None
    if cfg.zipf_s is not None:
        logp = zipf_log_popularity(cfg.E, cfg.zipf_s).astype(np.float32)
        logits += logp[expert_rank - 1][None, :]
    if cfg.hot_bias is not None:
        hot = int(np.nonzero(expert_rank == cfg.hot_rank)[0][0])
        logits[:, hot] += np.float32(cfg.hot_bias)

    x = bf16_from_f32(g_x.standard_normal((T, cfg.H), dtype=np.float32))
    y = None
    if with_y:
        y = bf16_from_f32(g_y.standard_normal((T * cfg.k, cfg.H), dtype=np.float32))
    return Workload(cfg=cfg, seed=seed, logits=np.ascontiguousarray(logits), x=x, y=y,
                    expert_rank=expert_rank, hot_expert=hot)
