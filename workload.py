"""Seeded synthetic inputs for compact decode attention.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic (no compaction, no quantisation, no attention).  Both the
CPU oracle and the GPU path are fed from here.

Workloads follow the FastDMS page ("FastDMS: 6.4X KV-cache compression running
faster than vLLM BF16/FP8"), memory-table paragraph: ctx_len 8192, gen_len 128,
concurrency c = 1 and 8, on Llama-3.2-1B and Qwen3-8B.  Only the attention
shapes of those models are reproduced; no weights, checkpoints or datasets are
used.  The keep mask stands in for the output of DMS's learned per-head
eviction predictor (page's DMS paragraph), which needs trained weights.

Recipe per (config, layer), all on the CPU with one torch.Generator seeded
``seed * 1000 + layer``, drawn in this order:
  1. keep rates r[B, Hkv]: a fixed rate, or U[lo, hi] per (sequence, head),
     times the layer's budget factor (1 for a flat budget; see
     ``layer_budget``), capped at 1
  2. keep bits [B, Hkv, T + S] ~ Bernoulli(r)          (uint8 0/1)
  3. K [B, T + S, Hkv, D] ~ N(0, 1) in float32, then V likewise
  4. outlier channels (optional): a fraction of the layer's Hkv*D channels,
     drawn without replacement separately for K and V, scaled x8
  5. K, V rounded to bfloat16 (round-to-nearest-even)
  6. q [S, B, Hq, D] ~ N(0, 1), rounded to bfloat16
Positions 0..T-1 are the prefill; position T+s is the token decoded at step s.
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    L: int            # layers
    B: int            # sequences (concurrency c)
    Hq: int           # query heads
    Hkv: int          # KV heads
    D: int            # head_dim
    T: int            # prefill length (ctx_len)
    S: int            # decode steps (gen_len)
    W: int            # always-kept recent window (staging)
    kv_dtype: str     # "bf16" or "fp8"
    keep_lo: float    # keep rate lower bound (== keep_hi for a fixed rate)
    keep_hi: float
    outlier_frac: float
    seed: int
    budget: str = "flat"   # "flat" or "pyramid" (keep rate falling with depth)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# The five workloads.  W = 256 for the Qwen shapes is a reading: the pages give
# a recent window only for the smaller model.
CONFIGS = {
    "tiny": Config("tiny", L=1, B=1, Hq=8, Hkv=2, D=64, T=512, S=1, W=64,
                   kv_dtype="bf16", keep_lo=1 / 6.4, keep_hi=1 / 6.4,
                   outlier_frac=0.0, seed=0),
    "llama_c1": Config("llama_c1", L=16, B=1, Hq=32, Hkv=8, D=64, T=8192, S=128,
                       W=256, kv_dtype="bf16", keep_lo=0.05, keep_hi=0.35,
                       outlier_frac=0.0, seed=1),
    "llama_c8": Config("llama_c8", L=16, B=8, Hq=32, Hkv=8, D=64, T=8192, S=128,
                       W=256, kv_dtype="fp8", keep_lo=0.05, keep_hi=0.35,
                       outlier_frac=0.0, seed=2),
    "qwen_c1": Config("qwen_c1", L=36, B=1, Hq=32, Hkv=8, D=128, T=8192, S=128,
                      W=256, kv_dtype="bf16", keep_lo=0.04, keep_hi=0.25,
                      outlier_frac=0.01, seed=3),
    "qwen_c8": Config("qwen_c8", L=36, B=8, Hq=32, Hkv=8, D=128, T=8192, S=128,
                      W=256, kv_dtype="fp8", keep_lo=0.04, keep_hi=0.25,
                      outlier_frac=0.01, seed=4),
}


def custom(name="custom", *, L=1, B=1, Hq=8, Hkv=2, D=64, T=256, S=1, W=16,
           kv_dtype="bf16", keep_lo=0.2, keep_hi=0.2, outlier_frac=0.0,
           seed=12345, budget="flat") -> Config:
    """A free-form config for property and edge-case tests."""
    return Config(name, L, B, Hq, Hkv, D, T, S, W, kv_dtype, keep_lo, keep_hi,
                  outlier_frac, seed, budget)


def pyramid(cfg: Config) -> Config:
    """The same workload with a per-layer budget that shrinks with depth.

    PyramidInfer page ("PyramidInfer: Pyramid KV Cache Compression for
    High-throughput LLM Inference"), abstract and technical-approach list:
    the number of keys and values that matter falls layer by layer, so
    deeper layers keep a shorter pivotal context.  The pages give no
    schedule; the reading here is a linear one that keeps the model's mean
    keep rate, so the flat and pyramid workloads store about the same bytes
    and differ only in how the rows are spread over the layers.
    """
    return dataclasses.replace(cfg, name=cfg.name + "_pyramid", budget="pyramid")


def layer_budget(cfg: Config, layer: int) -> float:
    """Factor on the keep rates of one layer: 1 for a flat budget; for the
    pyramid budget 1.5 at layer 0 falling linearly to 0.5 at layer L-1
    (mean 1 over the layers)."""
    if cfg.budget == "flat" or cfg.L == 1:
        return 1.0
    if cfg.budget != "pyramid":
        raise ValueError(f"unknown budget {cfg.budget!r}")
    return 1.5 - layer / (cfg.L - 1)


# The two c = 8 workloads with the pyramid budget.
CONFIGS.update({c.name: c for c in (pyramid(CONFIGS["llama_c8"]), pyramid(CONFIGS["qwen_c8"]))})


@dataclasses.dataclass
class Layer:
    """One layer's inputs, all CPU tensors.

    keep : uint8 [B, Hkv, T+S]   0/1 keep bit per position
    k, v : bfloat16 [B, T+S, Hkv, D]
    q    : bfloat16 [S, B, Hq, D]
    rate : float32 [B, Hkv]      the keep rate each head was drawn with
    """
    keep: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    q: torch.Tensor
    rate: torch.Tensor


def make_layer(cfg: Config, layer: int) -> Layer:
    g = torch.Generator().manual_seed(cfg.seed * 1000 + layer)
    B, Hkv, Hq, D, T, S = cfg.B, cfg.Hkv, cfg.Hq, cfg.D, cfg.T, cfg.S
    if cfg.keep_lo == cfg.keep_hi:
        rate = torch.full((B, Hkv), cfg.keep_lo, dtype=torch.float32)
    else:
        rate = cfg.keep_lo + (cfg.keep_hi - cfg.keep_lo) * torch.rand(
            (B, Hkv), generator=g, dtype=torch.float32)
    rate = (rate * layer_budget(cfg, layer)).clamp(max=1.0)
    keep = (torch.rand((B, Hkv, T + S), generator=g) < rate[..., None]).to(torch.uint8)
    k = torch.randn((B, T + S, Hkv, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, T + S, Hkv, D), generator=g, dtype=torch.float32)
    n_out = int(round(cfg.outlier_frac * Hkv * D))
    if n_out > 0:
        for x in (k, v):
            ch = torch.randperm(Hkv * D, generator=g)[:n_out]
            flat = x.view(B, T + S, Hkv * D)
            flat[:, :, ch] *= 8.0
    q = torch.randn((S, B, Hq, D), generator=g, dtype=torch.float32)
    return Layer(keep=keep, k=k.to(torch.bfloat16), v=v.to(torch.bfloat16),
                 q=q.to(torch.bfloat16), rate=rate)


def random_bf16(shape, seed: int, scale: float = 1.0) -> torch.Tensor:
    """N(0, scale^2) values rounded to bfloat16, from their own generator."""
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g)).to(torch.bfloat16)


def random_keep(shape, rate: float, seed: int) -> torch.Tensor:
    """Bernoulli(rate) keep bytes; a kept byte is drawn from 1..255 when the
    seed is odd, so that 'any nonzero byte keeps' is exercised."""
    g = torch.Generator().manual_seed(seed)
    kept = torch.rand(shape, generator=g) < rate
    if seed % 2:
        vals = torch.randint(1, 256, shape, generator=g, dtype=torch.int32)
    else:
        vals = torch.ones(shape, dtype=torch.int32)
    return torch.where(kept, vals, torch.zeros_like(vals)).to(torch.uint8)
