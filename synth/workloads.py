"""Seeded synthetic workloads for MoE row movement.

Five named shapes (token count T, hidden size H in bf16 elements, expert
count E, top-k k):

  tiny            T=128    H=1024  E=8    k=2  uniform routing, identity expert
  train           T=4096   H=7168  E=256  k=8  uniform routing, per-expert scale
  decode          T=128    H=7168  E=256  k=8  Zipf(1.2) routing, identity expert
  prefill         T=16384  H=7168  E=64   k=6  Zipf(1.0) routing, identity expert
  combine_stress  T=8192   H=4096  E=256  k=8  uniform routing, random expert
                                               outputs y, combine only

Recipe (seed = the shape's index 1..5 unless given;
``numpy.random.Generator(PCG64(seed))``; draws happen in this order):

1. x ~ N(0, 1) drawn in float32, rounded to bf16 by torch's conversion
   (round to nearest even).  Not drawn for ``combine_stress``.
2. routing: k distinct experts per token, drawn one after another without
   replacement with probability proportional to p_e, done as Gumbel-top-k
   (add an independent standard Gumbel to log p_e for every expert, keep the
   k largest keys in descending order, so column j is the j-th draw).
   Uniform routing uses p_e = 1/E; Zipf(s) uses p_e proportional to
   (e+1)^-s, so expert 0 is the most popular.
3. gate logits ~ N(0, sigma^2) float32 over the k chosen experts
   (sigma = 1, or sqrt(2) for ``combine_stress``), and the weights are their
   max-subtracted softmax in float32, column order kept.
4. ``train``: per-expert scale s_e ~ U(0.5, 1.5) float32.
   ``combine_stress``: y ~ N(0, 1) bf16 of shape [T*k, H], already in the
   expert-grouped row order.

Nothing here computes a layout, a dispatch or a combine.
"""

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    T: int
    H: int
    E: int
    k: int
    routing: str  # "uniform" | "zipf"
    zipf_s: Optional[float]
    logit_std: float
    expert: str  # "identity" | "scale" | "random_y"
    ops: str  # "dispatch+combine" | "combine"

    @property
    def rows(self):
        return self.T * self.k


CONFIGS = {
    c.name: c
    for c in [
        Config("tiny", 1, 128, 1024, 8, 2, "uniform", None, 1.0, "identity", "dispatch+combine"),
        Config("train", 2, 4096, 7168, 256, 8, "uniform", None, 1.0, "scale", "dispatch+combine"),
        Config("decode", 3, 128, 7168, 256, 8, "zipf", 1.2, 1.0, "identity", "dispatch+combine"),
        Config("prefill", 4, 16384, 7168, 64, 6, "zipf", 1.0, 1.0, "identity", "dispatch+combine"),
        Config("combine_stress", 5, 8192, 4096, 256, 8, "uniform", None, math.sqrt(2.0), "random_y", "combine"),
    ]
}


@dataclass
class Workload:
    config: Config
    seed: int
    topk_idx: np.ndarray  # int32 [T, k]
    topk_w: np.ndarray  # float32 [T, k]
    x: Optional[np.ndarray] = None  # uint16 [T, H] bf16 bits
    scales: Optional[np.ndarray] = None  # float32 [E]
    y: Optional[np.ndarray] = None  # uint16 [T*k, H] bf16 bits
    extra: dict = field(default_factory=dict)


def zipf_probs(E, s):
    """Finite Zipf popularity over E experts: p_e proportional to (e+1)^-s."""
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-float(s))
    return p / p.sum()


def _to_bf16_bits(f32):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _route(rng, T, E, k, probs):
    """Gumbel-top-k: k distinct experts per token, in draw order."""
    if k > E:
        raise ValueError("k must not exceed E")
    keys = rng.gumbel(size=(T, E))
    if probs is not None:
        keys = keys + np.log(probs)[None, :]
    order = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return np.ascontiguousarray(order.astype(np.int32))


def _softmax_f32(logits):
    logits = logits.astype(np.float32)
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m, dtype=np.float32)
    return (ex / ex.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


def make_workload(name, seed=None, **overrides):
    """Build the named workload; ``overrides`` may change T, H, E, k (for
    smaller parity cases of the same structure)."""
    cfg = CONFIGS[name]
    if overrides:
        cfg = replace(cfg, **overrides)
    if cfg.H % 8 != 0:
        raise ValueError("H must be a multiple of 8 (16-byte rows)")
    seed = cfg.index if seed is None else int(seed)
    rng = np.random.Generator(np.random.PCG64(seed))
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k

    x = None
    if cfg.ops != "combine":
        x = _to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))

    probs = zipf_probs(E, cfg.zipf_s) if cfg.routing == "zipf" else None
    topk_idx = _route(rng, T, E, k, probs)

    logits = rng.standard_normal((T, k), dtype=np.float32) * np.float32(cfg.logit_std)
    topk_w = _softmax_f32(logits)

    scales = None
    y = None
    if cfg.expert == "scale":
        scales = rng.uniform(0.5, 1.5, size=E).astype(np.float32)
    elif cfg.expert == "random_y":
        y = _to_bf16_bits(rng.standard_normal((T * k, H), dtype=np.float32))

    return Workload(cfg, seed, topk_idx, topk_w, x=x, scales=scales, y=y)


def algorithmic_bytes(T, H, k, E):
    """Bytes each step must move (1 GB = 1e9 B): dispatch reads each row once
    and writes it k times, combine reads k rows and writes one, layout reads
    the ids and writes two int32 maps plus counts and offsets."""
    row = 2 * H
    return {
        "layout": T * k * 4 + 2 * T * k * 4 + 8 * E + 4,
        "dispatch": T * row + T * k * row + T * k * 4,
        "combine": T * k * row + T * row + T * k * 8,
    }
