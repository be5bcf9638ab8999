"""Checks that pin the attention-side oracle (``oracle.attn_oracle``) to facts fixed outside it.

Each ``pin_*`` function takes the oracle module ``A`` and raises AssertionError when the oracle
disagrees with:

* the hand-worked example ``tests/golden/attn_worked_example.json`` (pencil and paper);
* brute-force scalar loops with exact summation (math.fsum) on tiny shapes;
* exact identities: every head listed gives the dense projections, computed here by one
  matrix product over the flattened heads (another route than the oracle's per-head loop); no
  head gives zeros; the output projection over disjoint head sets adds up;
* the closed form of the predictor's firing rate: for x ~ N(0, I) head h's logit is
  N(b_h, sigma_h^2), so it fires with probability Phi(b_h / sigma_h), which the generator sets
  to the target rate.

Shared by ``test_attn_oracle_pins.py`` (the oracle passes them) and
``test_attn_oracle_mutants.py`` (plausible mistakes planted in the oracle fail at least one).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from synth import attn as SA

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _worked():
    with open(os.path.join(GOLDEN, "attn_worked_example.json")) as f:
        ex = json.load(f)
    inp = {"w_a1": np.array(ex["w_a1"], np.float16), "w_a2": np.array(ex["w_a2"], np.float16),
           "bias_a": np.array(ex["bias_a"], np.float32), "w_qkv": np.array(ex["w_qkv"], np.float16),
           "w_o": np.array(ex["w_o"], np.float16)}
    return ex, inp, np.array(ex["x"], np.float16), np.array(ex["o"], np.float32)


def pin_attn_worked(A):
    ex, inp, x, o = _worked()
    lg = A.head_logits(x, inp["w_a1"], inp["w_a2"], inp["bias_a"])
    assert np.array_equal(lg, np.array(ex["logits"], float)), ("logits", lg)
    st = A.attn_step(inp, x, o)
    assert list(st["heads"]) == ex["active_heads"], ("heads", st["heads"])
    assert list(np.flatnonzero(st["band"])) == ex["band_heads"], ("band", st["band"])
    assert np.array_equal(st["qkv"], np.array(ex["qkv"], float)), ("qkv", st["qkv"])
    assert np.array_equal(st["y"], np.array(ex["y"], float)), ("y", st["y"])
    assert np.array_equal(A.qkv_heads(inp["w_qkv"], x, ex["active_heads"]), np.array(ex["qkv"], float))
    assert np.array_equal(A.out_heads(inp["w_o"], o, ex["active_heads"]), np.array(ex["y"], float))
    assert np.array_equal(A.qkv_dense(inp["w_qkv"], x), np.array(ex["qkv_dense"], float)), "qkv dense"
    assert np.array_equal(A.out_dense(inp["w_o"], o), np.array(ex["y_dense"], float)), "y dense"


def _brute(inp, x, o):
    w_a1, w_a2, b = (np.asarray(inp[k], np.float64) for k in ("w_a1", "w_a2", "bias_a"))
    d, r = w_a1.shape
    H = w_a2.shape[1]
    xf = [float(v) for v in x]
    z = [math.fsum(xf[k] * w_a1[k, j] for k in range(d)) for j in range(r)]
    lg = [math.fsum([z[j] * w_a2[j, h] for j in range(r)] + [b[h]]) for h in range(H)]
    heads = [h for h in range(H) if lg[h] > 0]
    wq = np.asarray(inp["w_qkv"], np.float64)
    wo = np.asarray(inp["w_o"], np.float64)
    dh = wq.shape[2]
    qkv = np.zeros((H, 3, dh))
    for h in heads:
        for m in range(3):
            for c in range(dh):
                qkv[h, m, c] = math.fsum(wq[h, m, c, k] * xf[k] for k in range(d))
    y = np.array([math.fsum(float(o[h, c]) * wo[h, c, j] for h in heads for c in range(dh))
                  for j in range(d)])
    return np.array(lg), heads, qkv, y


def pin_attn_bruteforce(A, seeds=(1, 2, 3)):
    for seed in seeds:
        cfg = SA.tiny(d=8, H=6, dh=3, r=3, T=3, seed=seed)
        inp = SA.make(cfg)
        for t in range(cfg.T):
            x, o = inp["x"][t], inp["o"][t]
            lg, heads, qkv, y = _brute(inp, x, o)
            st = A.attn_step(inp, x, o)
            assert np.allclose(st["logits"], lg, rtol=1e-12, atol=1e-12), (seed, t, "logits")
            assert list(st["heads"]) == heads, (seed, t, "heads", st["heads"], heads)
            assert np.allclose(st["qkv"], qkv, rtol=1e-12, atol=1e-13), (seed, t, "qkv")
            assert np.allclose(st["y"], y, rtol=1e-12, atol=1e-13), (seed, t, "y")


def pin_attn_identities(A, seed=5):
    cfg = SA.tiny(d=40, H=8, dh=5, r=6, T=2, seed=seed)
    inp = SA.make(cfg)
    x, o = inp["x"][0], inp["o"][0]
    H, dh, d = cfg.H, cfg.dh, cfg.d
    wq = np.asarray(inp["w_qkv"], np.float64).reshape(H * 3 * dh, d)
    wo = np.asarray(inp["w_o"], np.float64).reshape(H * dh, d)
    dense_qkv = (wq @ np.asarray(x, np.float64)).reshape(H, 3, dh)
    dense_y = np.asarray(o, np.float64).reshape(-1) @ wo
    assert np.allclose(A.qkv_dense(inp["w_qkv"], x), dense_qkv, rtol=1e-12, atol=1e-13), "qkv dense"
    assert np.allclose(A.out_dense(inp["w_o"], o), dense_y, rtol=1e-12, atol=1e-13), "y dense"
    assert np.array_equal(A.qkv_heads(inp["w_qkv"], x, []), np.zeros((H, 3, dh))), "qkv empty"
    assert np.array_equal(A.out_heads(inp["w_o"], o, []), np.zeros(d)), "y empty"
    s1, s2 = [0, 3, 5], [1, 2, 7]
    part = A.qkv_heads(inp["w_qkv"], x, s1)
    for h in range(H):
        want = dense_qkv[h] if h in s1 else np.zeros((3, dh))
        assert np.allclose(part[h], want, rtol=1e-12, atol=1e-13), ("qkv subset", h)
    y12 = A.out_heads(inp["w_o"], o, s1) + A.out_heads(inp["w_o"], o, s2)
    assert np.allclose(y12, A.out_heads(inp["w_o"], o, sorted(s1 + s2)), rtol=1e-12, atol=1e-13), "additive"


def pin_attn_rate_closed_form(A, tokens=20000, seed=9):
    cfg = SA.tiny(d=64, H=16, dh=4, r=8, T=1, seed=seed, mean_rate=0.4)
    inp = SA.make(cfg)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, cfg.d)).astype(np.float16)
    fired = A.head_logits(x, inp["w_a1"], inp["w_a2"], inp["bias_a"]) > 0
    emp = fired.mean(axis=0)
    # binomial standard error of each head's rate; 5 of them is far beyond chance
    se = np.sqrt(inp["rates"] * (1 - inp["rates"]) / tokens)
    assert np.all(np.abs(emp - inp["rates"]) < 5 * se + 2e-3), ("rates", emp, inp["rates"])


ALL_PINS = [pin_attn_worked, pin_attn_bruteforce, pin_attn_identities, pin_attn_rate_closed_form]
