"""Workload configurations for the predictor-gated sparse FFN.

Each configuration fixes the shapes, value distributions and activation-rate
law of one synthetic FFN layer.  The pages (PowerInfer, "Activation
Sparsity" / "Neuron Aware Operator" sections) describe the method on trained
LLMs with prompts drawn from conversational datasets; those are not available,
so seeded Gaussian weights at real model shapes and a power-law (Zipf) rate
law stand in for them.  Where the pages leave a parameter open, the field's
comment states the reading taken.

This module holds shapes and distribution parameters only: no arithmetic of
the method lives here.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class FFNConfig:
    name: str
    d: int                 # model width
    F: int                 # ffn width (number of neurons)
    r: int                 # predictor rank
    act: str               # "relu" or "reglu"
    wfmt: str              # "f16" or "i4g128"
    w_std: float           # std of the FFN weight draws (second N() parameter is a std)
    p_std: float           # std of the predictor weight draws
    zipf_s: float          # Zipf exponent of the per-neuron activation-rate law
    mean_rate: float       # target mean predicted-active fraction
    B: int                 # tokens decoded together (batch)
    T: int                 # decode steps
    seed: int = 0
    cap: float = 0.99      # upper clip of a Zipf rate
    hot_frac: float = 0.0  # fraction of neurons forced "hot" (c2 only)
    hot_rate: float = 0.0  # activation rate of the forced-hot neurons
    cold_cap: float = 0.0  # clip of the Zipf part when a hot set exists

    @property
    def m(self) -> int:
        """Number of FFN matrices touched per active neuron."""
        return 3 if self.act == "reglu" else 2

    @property
    def wbytes(self) -> float:
        """Bytes per stored weight (int4 adds one fp16 scale per 128)."""
        return 2.0 if self.wfmt == "f16" else 0.5 + 2.0 / 128.0

    @property
    def mask_words(self) -> int:
        return (self.F + 31) // 32

    def with_(self, **kw) -> "FFNConfig":
        return replace(self, **kw)


# Tiny ReLU FFN: d=1024, ffn=4096, rank 128, Zipf(1.1), ~10% active, 64 tokens.
C1 = FFNConfig("c1_tiny_relu", d=1024, F=4096, r=128, act="relu", wfmt="f16",
               w_std=0.02, p_std=0.05, zipf_s=1.1, mean_rate=0.10, B=1, T=64)

# LLaMA-7B-shaped ReGLU FFN.  "5% hot with rate > 0.8" cannot coexist with a
# single clipped Zipf(1.2) at a 10% mean (only ~3.4% of neurons would exceed
# 0.8), so a random 5% is pinned at rate 0.90 and the rest follow a Zipf(1.2)
# capped at 0.80, scaled so the overall mean is 10%.
C2 = FFNConfig("c2_llama7b_reglu", d=4096, F=11008, r=256, act="reglu", wfmt="f16",
               w_std=0.02, p_std=0.05, zipf_s=1.2, mean_rate=0.10, B=1, T=256,
               hot_frac=0.05, hot_rate=0.90, cold_cap=0.80)

# OPT-30B-shaped ReLU FFN, Zipf(1.3), ~5% active.
C3 = FFNConfig("c3_opt30b_relu", d=7168, F=28672, r=512, act="relu", wfmt="f16",
               w_std=0.015, p_std=0.05, zipf_s=1.3, mean_rate=0.05, B=1, T=256)

# Falcon-40B-shaped ReLU FFN, batch-32 decode on the union of the token masks.
# The Zipf exponent and weight std are not given: 1.2 and N(0, 0.02) are used.
C4 = FFNConfig("c4_falcon40b_relu_b32", d=8192, F=32768, r=512, act="relu", wfmt="f16",
               w_std=0.02, p_std=0.05, zipf_s=1.2, mean_rate=0.08, B=32, T=64)

# LLaMA-70B-shaped ReGLU FFN with weight-only int4 (group 128 along d).
C5 = FFNConfig("c5_llama70b_reglu_int4", d=8192, F=28672, r=1024, act="reglu", wfmt="i4g128",
               w_std=0.01, p_std=0.05, zipf_s=1.2, mean_rate=0.10, B=1, T=128)

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5)}
ORDER = [C1, C2, C3, C4, C5]
SHORT = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}


def get(name: str) -> FFNConfig:
    if name in SHORT:
        return SHORT[name]
    return CONFIGS[name]


def tiny(act: str = "relu", wfmt: str = "f16", *, d: int = 384, F: int = 1000, r: int = 40,
         B: int = 1, T: int = 4, seed: int = 7, mean_rate: float = 0.2,
         zipf_s: float = 1.1) -> FFNConfig:
    """A small configuration whose sizes leave ragged tails against the kernels' tiles.

    Defaults: d=384 (not a multiple of 512), F=1000 (not a multiple of 32 or 64),
    r=40 (not a power of two).  int4 needs d to be a multiple of 128.
    """
    return FFNConfig(f"tiny_{act}_{wfmt}_d{d}_F{F}_r{r}_B{B}", d=d, F=F, r=r, act=act, wfmt=wfmt,
                     w_std=0.02, p_std=0.05, zipf_s=zipf_s, mean_rate=mean_rate, B=B, T=T,
                     seed=seed)
