"""Seeded synthetic inputs for the MoE-layer hot path (routing, permute + MX
quantization, grouped GEMMs, weighted combine).

This module is shared by the tests, the CPU oracle and the benchmark, and so it
holds none of the method's arithmetic: it only draws random numbers and stores
them in the dtypes the operators take (bf16 activations and weight masters,
int32 expert ids, fp32 gate weights). Quantizing the weight masters to MXFP8 is
the caller's job: the oracle's quantizer in tests, the library's own quantizer
on the GPU in the benchmark.

Workloads (shapes from the MegaMoE "A8W8-FP" scenario and the MoeInitRoutingV3
large-batch template):

* ``tiny``     64 tokens, hidden 256, intermediate 128, 8 experts, topK 2, E4M3
* ``decode``   128 tokens, hidden 7168, intermediate 2048, 256 experts, topK 8, E4M3
* ``prefill``  8192 tokens, same layer, plus one shared expert over all tokens
* ``skewed``   4096 tokens, hidden 4096, intermediate 1536, 128 experts, topK 6,
               Zipf(1.2) expert popularity, E5M2, activations N(0, 2)
* ``routing``  32768 tokens, hidden 7168, 256 experts, topK 8, active expert
               range [32, 64), scatter row index, count histogram, E4M3

Distributions: activations are N(0, sigma) rounded to bf16 (sigma is a standard
deviation); weight masters are N(0, 1/sqrt(fan_in)) rounded to bf16, fan_in being
the contraction length (hidden for W1, intermediate for W2); expert ids are K
distinct ids per token, uniform, or drawn without replacement with
p(rank r) proportional to r^-s; gate weights are the softmax of K N(0,1) logits.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = [
    "LayerConfig",
    "CONFIGS",
    "config",
    "expert_ids",
    "gate_weights",
    "activations",
    "weight_master",
    "derive_seed",
]


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    tokens: int          # N (BS)
    hidden: int          # H
    inter: int           # I (intermediateHidden); 0 for routing-only workloads
    experts: int         # E (all local on one GPU)
    topk: int            # K
    fmt: str             # "e4m3" or "e5m2"
    sigma: float = 1.0   # std of the activations
    shared: int = 0      # shared experts over all tokens
    routing: str = "uniform"   # "uniform" or "zipf"
    zipf_s: float = 1.2
    active: tuple | None = None  # active expert range [start, end)
    seed: int = 1000

    @property
    def flat(self) -> int:
        return self.tokens * self.topk

    @property
    def active_range(self) -> tuple:
        return self.active if self.active is not None else (0, self.experts)


CONFIGS = {
    "tiny": LayerConfig("tiny", 64, 256, 128, 8, 2, "e4m3", seed=1000),
    "decode": LayerConfig("decode", 128, 7168, 2048, 256, 8, "e4m3", seed=1001),
    "prefill": LayerConfig("prefill", 8192, 7168, 2048, 256, 8, "e4m3", shared=1, seed=1002),
    "skewed": LayerConfig("skewed", 4096, 4096, 1536, 128, 6, "e5m2", sigma=2.0,
                          routing="zipf", seed=1003),
    "routing": LayerConfig("routing", 32768, 7168, 0, 256, 8, "e4m3", active=(32, 64),
                           seed=1004),
}


def config(name: str, **overrides) -> LayerConfig:
    """A named workload, optionally with fields replaced (smaller test shapes)."""
    return dataclasses.replace(CONFIGS[name], **overrides)


_TAGS = {"ids": 1, "gate": 2, "x": 3, "w1": 4, "w2": 5, "sw1": 6, "sw2": 7, "w2g": 8, "sw2g": 9}


def derive_seed(seed: int, tag: str, index: int = 0) -> int:
    """SplitMix64 finaliser over (seed, tag, index): independent streams per tensor."""
    z = (seed * 0x9E3779B97F4A7C15 + _TAGS[tag] * 0xBF58476D1CE4E5B9 + index * 0x94D049BB133111EB)
    z &= (1 << 64) - 1
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & ((1 << 64) - 1)
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & ((1 << 64) - 1)
    z ^= z >> 31
    return z & ((1 << 63) - 1)


def expert_ids(cfg: LayerConfig) -> np.ndarray:
    """int32 [N, K]: K distinct expert ids per token.

    uniform: a uniformly random K-subset in random order (argsort of iid keys).
    zipf:    sequential draws without replacement with p(rank r) ~ r^-s, expert id
             r - 1, realised with the Gumbel-top-K identity (sorting log p plus
             Gumbel noise and keeping the first K gives the same law as drawing K
             times without replacement, renormalising after each draw).
    """
    rng = np.random.default_rng(derive_seed(cfg.seed, "ids"))
    n, e, k = cfg.tokens, cfg.experts, cfg.topk
    ids = np.empty((n, k), dtype=np.int32)
    chunk = 4096
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        if cfg.routing == "uniform":
            keys = rng.random((hi - lo, e))
        elif cfg.routing == "zipf":
            logp = -cfg.zipf_s * np.log(np.arange(1, e + 1, dtype=np.float64))
            keys = -(logp[None, :] + rng.gumbel(size=(hi - lo, e)))
        else:
            raise ValueError(cfg.routing)
        ids[lo:hi] = np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    return ids


def gate_weights(cfg: LayerConfig) -> np.ndarray:
    """fp32 [N, K]: softmax over the K selected experts of N(0,1) logits."""
    rng = np.random.default_rng(derive_seed(cfg.seed, "gate"))
    logits = rng.standard_normal((cfg.tokens, cfg.topk))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def activations(cfg: LayerConfig) -> torch.Tensor:
    """bf16 [N, H] on the CPU: N(0, sigma) drawn in fp32, rounded to bf16 (RNE)."""
    rng = np.random.default_rng(derive_seed(cfg.seed, "x"))
    out = torch.empty((cfg.tokens, cfg.hidden), dtype=torch.bfloat16)
    rows = max(1, (1 << 24) // max(1, cfg.hidden))
    for lo in range(0, cfg.tokens, rows):
        hi = min(cfg.tokens, lo + rows)
        a = rng.standard_normal((hi - lo, cfg.hidden), dtype=np.float32) * np.float32(cfg.sigma)
        out[lo:hi] = torch.from_numpy(a).to(torch.bfloat16)
    return out


def weight_master(cfg: LayerConfig, which: str, expert: int, device="cpu") -> torch.Tensor:
    """bf16 master weights of one expert, in the stored (out, in) orientation.

    which: "w1" -> [2I, H] (gate rows [0, I), up rows [I, 2I)), fan_in H
           "w2" -> [H, I], fan_in I
           "w2g" -> [H, 2I], fan_in 2I (weight2 of a gelu layer, whose A is 2I wide)
           "sw1"/"sw2"/"sw2g" -> the same for shared expert ``expert``.
    Drawn with torch's generator on ``device`` seeded per (config, tensor, expert),
    so any single expert can be regenerated on its own. CPU and GPU generators give
    different (equally valid) draws; a given device always gives the same ones.
    """
    h, i = cfg.hidden, cfg.inter
    shape, fan_in = {"w1": ((2 * i, h), h), "w2": ((h, i), i), "w2g": ((h, 2 * i), 2 * i),
                     "sw1": ((2 * i, h), h), "sw2": ((h, i), i), "sw2g": ((h, 2 * i), 2 * i)}[which]
    gen = torch.Generator(device=device)
    gen.manual_seed(derive_seed(cfg.seed, which, expert))
    w = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    w.mul_(1.0 / math.sqrt(fan_in))
    return w.to(torch.bfloat16)
