"""Seeded synthetic inputs for the predictor-gated sparse FFN.

This module is shared by the oracle-side tests and the GPU side: it draws
weights, token activations and the per-neuron predictor bias, and packs int4
weights.  It contains none of the method's arithmetic (no predictor
evaluation, no thresholding, no compaction, no FFN); the only linear algebra
here sizes the bias so the *predicted* activation rates follow the intended
power law.

Recipe (PowerInfer, "Activation Sparsity" section: a few hot neurons fire on
most inputs, the cold majority fire rarely -- a power law):

* Every array is drawn from its own child stream of
  ``numpy.random.SeedSequence(seed)``, so any array can be regenerated alone.
* Weights: fp32 standard normal times the configured std, rounded to fp16
  (round-to-nearest-even).  int4 weights are quantised from those fp32 draws.
* Tokens: x_t ~ N(0, I) independently per step (no residual recurrence), fp16.
* Rates: a seeded permutation deals Zipf ranks 1..F to neurons; rank k gets
  p_k = min(c * k**-s, cap) with c found by bisection so mean(p) hits the
  target.  With a hot set (c2), a random hot_frac of neurons is pinned at
  hot_rate and the rest follow the capped Zipf, scaled so the overall mean is
  the target.
* Bias: the predictor logit of neuron i is l_i = x W_p1[:, .] W_p2[:, i] + b_i.
  For x ~ N(0, I) it is Gaussian with mean b_i and variance
  sigma_i^2 = W_p2[:, i]^T (W_p1^T W_p1) W_p2[:, i].  Choosing
  b_i = sigma_i * Phi^-1(p_i) makes P(l_i > 0) = p_i exactly.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
from scipy.special import ndtri

from .configs import FFNConfig

GEN_VERSION = 1
_STREAMS = ("perm", "w_p1", "w_p2", "w_gate", "w_up", "w_down", "x", "x_cal")
GROUP = 128  # int4 group size along d


def _rngs(seed: int) -> dict:
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {n: np.random.default_rng(k) for n, k in zip(_STREAMS, kids)}


def _normal_f16(rng, shape, std) -> np.ndarray:
    """fp32 N(0,1) draws times std, rounded to fp16; built in row chunks to bound memory."""
    out = np.empty(shape, dtype=np.float16)
    rows = shape[0]
    step = max(1, (1 << 22) // max(1, int(np.prod(shape[1:]))))
    blk = np.empty((min(step, rows),) + tuple(shape[1:]), dtype=np.float32)   # reused scratch
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        b = blk[:r1 - r0]
        rng.standard_normal(dtype=np.float32, out=b)
        b *= np.float32(std)
        out[r0:r1] = b
    return out


def zipf_rates(n: int, s: float, mean: float, cap: float) -> np.ndarray:
    """Rates p_k = min(c k^-s, cap) for ranks k = 1..n, with c chosen so mean(p) = mean."""
    if not (0.0 < mean < cap <= 1.0):
        raise ValueError(f"infeasible rate law: mean={mean} cap={cap}")
    base = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    lo, hi = 0.0, cap / base[-1]  # hi saturates every rank at cap
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(c * base, cap).mean() < mean:
            lo = c
        else:
            hi = c
    return np.minimum(0.5 * (lo + hi) * base, cap)


def neuron_rates(cfg: FFNConfig, perm: np.ndarray) -> np.ndarray:
    """Per-neuron target activation rates, dealt to neurons by the permutation."""
    F = cfg.F
    p = np.empty(F, dtype=np.float64)
    if cfg.hot_frac > 0:
        n_hot = int(round(cfg.hot_frac * F))
        hot, cold = perm[:n_hot], perm[n_hot:]
        cold_mean = (cfg.mean_rate * F - cfg.hot_rate * n_hot) / (F - n_hot)
        p[hot] = cfg.hot_rate
        p[cold] = zipf_rates(F - n_hot, cfg.zipf_s, cold_mean, cfg.cold_cap)
    else:
        p[perm] = zipf_rates(F, cfg.zipf_s, cfg.mean_rate, cfg.cap)
    return p


def logit_sigma(w_p1: np.ndarray, w_p2: np.ndarray) -> np.ndarray:
    """Std of each predictor logit for x ~ N(0, I), from the stored fp16 weights (f64)."""
    a = w_p1.astype(np.float64)
    g = a.T @ a                        # r x r Gram matrix
    p = w_p2.astype(np.float64)        # [r, F]
    return np.sqrt(np.einsum("jf,jf->f", g @ p, p))


def quantize_int4_g128(w: np.ndarray):
    """Symmetric round-to-nearest int4, one fp16 scale per 128 weights along the row.

    s = fp16(absmax / 7); q = clip(rint(w / s), -8, 7) (half to even); absmax = 0 gives
    s = 0, q = 0.  Stored nibble u = q + 8, two per byte, the even column in the low
    nibble.  Returns (packed u8 [rows, d/2], scales fp16 [rows, d/128]).
    """
    rows, d = w.shape
    if d % GROUP:
        raise ValueError("int4 rows need d % 128 == 0")
    packed = np.empty((rows, d // 2), dtype=np.uint8)
    scales = np.empty((rows, d // GROUP), dtype=np.float16)
    step = max(1, (1 << 20) // d)
    # scratch reused across row blocks (large temporaries would be page-faulted in afresh
    # for every block); the arithmetic is the one stated above, element by element
    q = np.empty((step, d // GROUP, GROUP), dtype=np.float32)
    u = np.empty((step, d), dtype=np.uint8)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        n = r1 - r0
        g = w[r0:r1].astype(np.float32, copy=False).reshape(n, d // GROUP, GROUP)
        qn = q[:n]
        np.abs(g, out=qn)
        s16 = (qn.max(axis=2) / np.float32(7.0)).astype(np.float16)
        s = s16.astype(np.float32)[..., None]
        pos = s > 0
        with np.errstate(divide="ignore", invalid="ignore"):
            np.divide(g, np.where(pos, s, np.float32(1)), out=qn)
        np.rint(qn, out=qn)
        np.multiply(qn, pos, out=qn)
        np.clip(qn, -8, 7, out=qn)
        qn += 8
        un = u[:n]
        un[...] = qn.reshape(n, d)
        packed[r0:r1] = un[:, 0::2] | (un[:, 1::2] << 4)
        scales[r0:r1] = s16
    return packed, scales


def quantize_int8_g128(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric int8 weight-only quantization with one fp16 scale per 128 columns:
    s = max|w| / 127 over the group (rounded to fp16), q = clip(rint(w / s), -127, 127).
    Returns (q int8 [rows, cols], scales fp16 [rows, cols/128])."""
    rows, cols = w.shape
    if cols % GROUP:
        raise ValueError("int8 rows need cols % 128 == 0")
    g = np.asarray(w, np.float32).reshape(rows, cols // GROUP, GROUP)
    s16 = (np.abs(g).max(axis=2) / np.float32(127.0)).astype(np.float16)
    s = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(g / np.where(s > 0, s, 1)), 0)
    return np.clip(q, -127, 127).astype(np.int8).reshape(rows, cols), s16


def predictor_int8(inputs: dict) -> dict:
    """The layer's predictor factors, transposed (one row per output) and quantized to int8
    group-128: q_p1t [r, d], s_p1t [r, d/128], q_p2t [F, r], s_p2t [F, r/128]."""
    q1, s1 = quantize_int8_g128(np.ascontiguousarray(inputs["w_p1"].T))
    q2, s2 = quantize_int8_g128(np.ascontiguousarray(inputs["w_p2"].T))
    return dict(q_p1t=q1, s_p1t=s1, q_p2t=q2, s_p2t=s2)


def _normal_i4(rng, shape, std):
    rows, d = shape
    packed = np.empty((rows, d // 2), dtype=np.uint8)
    scales = np.empty((rows, d // GROUP), dtype=np.float16)
    step = max(1, (1 << 22) // d)
    blk = np.empty((step, d), dtype=np.float32)         # reused: draws are sequential either way
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        b = blk[:r1 - r0]
        rng.standard_normal(dtype=np.float32, out=b)
        b *= np.float32(std)
        packed[r0:r1], scales[r0:r1] = quantize_int4_g128(b)
    return packed, scales


def make(cfg: FFNConfig, *, ffn: bool = True, tokens: bool = True) -> dict:
    """Draw one configuration's inputs.

    Keys: x fp16 [T, B, d]; w_p1 fp16 [d, r]; w_p2 fp16 [r, F]; bias fp32 [F];
    rates f64 [F] (target P(logit > 0)); sigma f64 [F] (logit std);
    fp16 FFN: w_up, w_down and (ReGLU) w_gate fp16 [F, d], all neuron-major;
    int4 FFN: q_up/q_down/(q_gate) u8 [F, d/2] and s_up/s_down/(s_gate) fp16 [F, d/128].
    """
    st = _rngs(cfg.seed)
    perm = st["perm"].permutation(cfg.F)
    w_p1 = _normal_f16(st["w_p1"], (cfg.d, cfg.r), cfg.p_std)
    w_p2 = _normal_f16(st["w_p2"], (cfg.r, cfg.F), cfg.p_std)
    rates = neuron_rates(cfg, perm)
    sigma = logit_sigma(w_p1, w_p2)
    bias = (sigma * ndtri(rates)).astype(np.float32)
    out = dict(cfg=cfg, perm=perm, w_p1=w_p1, w_p2=w_p2, bias=bias, rates=rates, sigma=sigma)
    if ffn:
        if cfg.wfmt not in ("f16", "i4g128"):
            raise ValueError(cfg.wfmt)
        mats = ("gate", "up", "down") if cfg.act == "reglu" else ("up", "down")

        def draw(name):
            rng = st["w_" + name]
            if cfg.wfmt == "f16":
                return {"w_" + name: _normal_f16(rng, (cfg.F, cfg.d), cfg.w_std)}
            q, sc = _normal_i4(rng, (cfg.F, cfg.d), cfg.w_std)
            return {"q_" + name: q, "s_" + name: sc}

        # every matrix has its own stream, so drawing them side by side (numpy fills without
        # holding the interpreter lock) gives the same arrays as drawing them in turn
        with ThreadPoolExecutor(max_workers=len(mats)) as ex:
            for part in ex.map(draw, mats):
                out.update(part)
    if tokens:
        out["x"] = _normal_f16(st["x"], (cfg.T, cfg.B, cfg.d), 1.0)
    return out


def expected_union(rates: np.ndarray, B: int) -> float:
    """Expected size of the OR of B independent token masks with these rates."""
    return float(np.sum(1.0 - (1.0 - rates) ** B))


def calibration_x(cfg: FFNConfig, n: int) -> np.ndarray:
    """n calibration tokens fp16 [n, d], x ~ N(0, 1), from a stream of their own (no token of
    the workload's stream): the profiling run behind a neuron placement."""
    return _normal_f16(_rngs(cfg.seed)["x_cal"], (n, cfg.d), 1.0)
