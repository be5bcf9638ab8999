"""Seeded synthetic inputs for the attention side of the layer: its predictor and the
head-major q/k/v and output projections.

Shared by the oracle-side tests and the GPU side; it holds none of the method's arithmetic
(no predictor evaluation, no thresholding, no projection).  The pages give no shapes, rank or
sparsity for the attention predictor ("Adaptive Sparsity Predictors" only says every layer has
one for the self-attention block next to the MLP one), so the workloads take multi-head
attention at the shapes of the models the FFN workloads follow and these readings:

* heads fire independently per token with per-head rates following the FFN recipe's power law
  (a seeded permutation deals Zipf ranks 1..H; rank k gets min(c k^-s, cap), mean 0.5);
* the predictor rank is 128 (LLaMA-7B shape) or 256 (OPT-30B shape), drawn N(0, 0.05^2) like
  the MLP predictor, with each head's bias b_h = sigma_h Phi^-1(p_h) so that P(l_h > 0) = p_h
  for x ~ N(0, I) (the same sizing the FFN generator uses);
* projection weights N(0, std^2) rounded to fp16, head-major: w_qkv [H, 3, d_head, d],
  w_o [H, d_head, d];
* tokens x ~ N(0, I) in fp16; the attention output the projection reads, o [T, H, d_head],
  ~ N(0, 1) in fp32 (it stands in for the attention core, which is outside this path).

Every array comes from its own child stream of SeedSequence(seed).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
from scipy.special import ndtri

from .gen import _normal_f16, logit_sigma, zipf_rates

_STREAMS = ("perm", "w_a1", "w_a2", "w_qkv", "w_o", "x", "o")


@dataclass(frozen=True)
class AttnConfig:
    name: str
    d: int                 # model width
    H: int                 # heads
    dh: int                # head width
    r: int                 # attention predictor rank
    w_std: float           # std of the projection weight draws
    p_std: float = 0.05    # std of the predictor weight draws
    zipf_s: float = 1.1    # Zipf exponent of the per-head rate law
    mean_rate: float = 0.5 # target mean fraction of heads predicted active
    cap: float = 0.99
    T: int = 16            # decode steps
    seed: int = 0

    def with_(self, **kw) -> "AttnConfig":
        return replace(self, **kw)


# LLaMA-7B-shaped multi-head attention: d = 4096, 32 heads of 128.
A2 = AttnConfig("a2_llama7b_attn", d=4096, H=32, dh=128, r=128, w_std=0.02, T=64, seed=102)
# OPT-30B-shaped multi-head attention: d = 7168, 56 heads of 128.
A3 = AttnConfig("a3_opt30b_attn", d=7168, H=56, dh=128, r=256, w_std=0.015, T=64, seed=103)

CONFIGS = {c.name: c for c in (A2, A3)}
SHORT = {"a2": A2, "a3": A3}


def get(name: str) -> AttnConfig:
    return SHORT[name] if name in SHORT else CONFIGS[name]


def tiny(*, d: int = 200, H: int = 8, dh: int = 24, r: int = 16, T: int = 4, seed: int = 7,
         mean_rate: float = 0.5) -> AttnConfig:
    """A small configuration: d and the head widths leave ragged tails against 64 and 512."""
    return AttnConfig(f"tiny_attn_d{d}_H{H}_dh{dh}_r{r}", d=d, H=H, dh=dh, r=r, w_std=0.05, T=T,
                      seed=seed, mean_rate=mean_rate)


def make(cfg: AttnConfig) -> dict:
    """Keys: x fp16 [T, d]; o fp32 [T, H, dh]; w_a1 fp16 [d, r]; w_a2 fp16 [r, H]; bias_a fp32
    [H]; rates f64 [H]; w_qkv fp16 [H, 3, dh, d]; w_o fp16 [H, dh, d]."""
    kids = np.random.SeedSequence(cfg.seed).spawn(len(_STREAMS))
    st = {n: np.random.default_rng(k) for n, k in zip(_STREAMS, kids)}
    perm = st["perm"].permutation(cfg.H)
    w_a1 = _normal_f16(st["w_a1"], (cfg.d, cfg.r), cfg.p_std)
    w_a2 = _normal_f16(st["w_a2"], (cfg.r, cfg.H), cfg.p_std)
    rates = np.empty(cfg.H)
    rates[perm] = zipf_rates(cfg.H, cfg.zipf_s, cfg.mean_rate, cfg.cap)
    bias_a = (logit_sigma(w_a1, w_a2) * ndtri(rates)).astype(np.float32)
    return dict(cfg=cfg, w_a1=w_a1, w_a2=w_a2, bias_a=bias_a, rates=rates,
                w_qkv=_normal_f16(st["w_qkv"], (cfg.H, 3, cfg.dh, cfg.d), cfg.w_std),
                w_o=_normal_f16(st["w_o"], (cfg.H, cfg.dh, cfg.d), cfg.w_std),
                x=_normal_f16(st["x"], (cfg.T, cfg.d), 1.0),
                o=st["o"].standard_normal((cfg.T, cfg.H, cfg.dh), dtype=np.float32))
