"""Checks that pin the CPU oracle to facts fixed outside the oracle itself.

Each ``pin_*`` function takes the oracle module ``O`` and raises AssertionError
when the oracle disagrees with:

* hand-worked examples (``tests/golden/*.json``, derived with pencil and paper);
* brute-force scalar loops with exact summation (math.fsum) on tiny shapes;
* exact identities of the masked FFN: the true-support mask and the all-ones
  mask both reproduce the dense FFN, masks over disjoint neuron sets add up,
  an empty mask gives exactly zero (PowerInfer, "Neuron-aware Operator": the
  skipped neurons contribute nothing);
* the closed form of the predictor's firing rate: for x ~ N(0, I) the logit
  of neuron i is N(b_i, sigma_i^2), so it fires with probability
  Phi(b_i / sigma_i), which the generator sets to the Zipf target p_i;
* the int4 codec's round-trip error bound (LLM Runtime page, "04 Accuracy":
  round-to-nearest quantisation).

The functions are shared by ``test_oracle_pins.py`` (the oracle passes them)
and ``test_oracle_mutants.py`` (plausible mistakes planted in the oracle fail
at least one of them).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from synth import configs, gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _ffn_inputs(ex, act):
    arrays = {"w_up": np.array(ex["w_up"], np.float16), "w_down": np.array(ex["w_down"], np.float16)}
    if act == "reglu":
        arrays["w_gate"] = np.array(ex["w_gate"], np.float16)
    return arrays


def pin_worked_example(O):
    ex = _load("worked_example.json")
    x = np.array(ex["x"], np.float16)
    lg = O.predictor_logits(x, np.array(ex["w_p1"], np.float16), np.array(ex["w_p2"], np.float16),
                            np.array(ex["bias"], np.float32))
    assert np.array_equal(lg, np.array(ex["logits"], float)), ("logits", lg)
    act = O.predicted_active(lg, O.logit_threshold(0.5))
    idx = O.compact(act)
    assert list(idx) == ex["active_idx"], ("idx", idx)
    assert list(O.mask_words(act)) == ex["mask_words"], "mask words"
    for a in ("relu", "reglu"):
        W = O.Weights(a, "f16", _ffn_inputs(ex, a))
        y = O.ffn_neurons(W, x, idx)
        assert np.array_equal(y, np.array(ex[a + "_y_pred"], float)), (a, "pred", y)
        yd = O.ffn_dense(W, x)
        assert np.array_equal(yd, np.array(ex[a + "_y_dense"], float)), (a, "dense", yd)
        pa = O.preact(W, x)
        assert np.array_equal(pa["a"], np.array(ex["a"], float)), "preact a"
        if a == "reglu":
            assert np.array_equal(pa["g"], np.array(ex["g"], float)), "preact g"
            support = np.flatnonzero(np.array(ex["g"], float) > 0)
        else:
            support = np.flatnonzero(np.array(ex["a"], float) > 0)
        ys = O.ffn_neurons(W, x, support)
        assert np.array_equal(ys, yd), (a, "true support", ys)


def _int4_rows(spec_bytes, spec_scales, F, d):
    q = np.full((F, d // 2), 0x88, np.uint8)
    for r, b, v in spec_bytes:
        q[r, b] = v
    return q, np.array(spec_scales, np.float16)


def pin_int4_worked(O):
    ex = _load("int4_worked_example.json")
    F, d = ex["F"], ex["d"]
    qu, su = _int4_rows(ex["up_bytes"], ex["up_scales"], F, d)
    qd, sd = _int4_rows(ex["down_bytes"], ex["down_scales"], F, d)
    Wu = O.unpack_int4(qu, su)
    want = np.zeros((F, d))
    for r, k, v in ex["up_nonzero"]:
        want[r, k] = v
    assert np.array_equal(Wu, want), "int4 unpack"
    x = np.zeros(d, np.float16)
    for k, v in ex["x_nonzero"]:
        x[k] = v
    assert np.array_equal(Wu @ x.astype(float), np.array(ex["up_dot"])), "int4 dot"
    W = O.Weights("relu", "i4g128", {"q_up": qu, "s_up": su, "q_down": qd, "s_down": sd})
    y = O.ffn_neurons(W, x, np.arange(F))
    wy = np.zeros(d)
    for k, v in ex["relu_y_nonzero"]:
        wy[k] = v
    assert np.array_equal(y, wy), "int4 relu ffn"


# ----------------------------------------------------------------------------- brute force
def _brute_logits(x, w_p1, w_p2, b):
    d, r = w_p1.shape
    F = w_p2.shape[1]
    z = [math.fsum(float(x[k]) * float(w_p1[k, j]) for k in range(d)) for j in range(r)]
    return np.array([math.fsum([z[j] * float(w_p2[j, i]) for j in range(r)] + [float(b[i])])
                     for i in range(F)])


def _brute_weight(arr, name, i, k, wfmt):
    if wfmt == "f16":
        return float(arr["w_" + name][i, k])
    byte = int(arr["q_" + name][i, k // 2])
    u = (byte >> (4 * (k % 2))) & 15
    return (u - 8) * float(arr["s_" + name][i, k // 128])


def _brute_ffn(arr, act, wfmt, x, idx, d):
    y = [[] for _ in range(d)]
    for i in idx:
        a = math.fsum(_brute_weight(arr, "up", i, k, wfmt) * float(x[k]) for k in range(d))
        if act == "relu":
            h = a if a > 0 else 0.0
        else:
            g = math.fsum(_brute_weight(arr, "gate", i, k, wfmt) * float(x[k]) for k in range(d))
            h = (g if g > 0 else 0.0) * a
        for j in range(d):
            y[j].append(h * _brute_weight(arr, "down", i, j, wfmt))
    return np.array([math.fsum(t) for t in y])


def _tiny_inputs(act, wfmt, seed, d, F, r, mean_rate=0.3):
    cfg = configs.tiny(act, wfmt, d=d, F=F, r=r, T=2, seed=seed, mean_rate=mean_rate)
    return gen.make(cfg)


def pin_bruteforce(O, seeds=(1, 2)):
    for seed in seeds:
        for act, wfmt, d in (("relu", "f16", 8), ("reglu", "f16", 8), ("reglu", "i4g128", 128)):
            inp = _tiny_inputs(act, wfmt, seed, d=d, F=16, r=2)
            x = inp["x"][0, 0]
            lg = O.predictor_logits(x, inp["w_p1"], inp["w_p2"], inp["bias"])
            bl = _brute_logits(x, inp["w_p1"], inp["w_p2"], inp["bias"])
            assert np.allclose(lg, bl, rtol=1e-12, atol=1e-12), (act, wfmt, "logits")
            idx = O.compact(O.predicted_active(lg))
            want_idx = [i for i in range(16) if bl[i] > 0]
            assert list(idx) == want_idx, (act, wfmt, "idx", idx, want_idx)
            W = O.Weights(act, wfmt, inp)
            for sel in (idx, np.arange(16)):
                y = O.ffn_neurons(W, x, sel)
                yb = _brute_ffn(inp, act, wfmt, x, list(sel), d)
                assert np.allclose(y, yb, rtol=1e-11, atol=1e-12), (act, wfmt, "ffn")


# ----------------------------------------------------------------------------- identities
def _identity_cases(seed=3):
    for act, wfmt, d in (("relu", "f16", 256), ("reglu", "f16", 256), ("relu", "i4g128", 256),
                         ("reglu", "i4g128", 256)):
        yield act, wfmt, _tiny_inputs(act, wfmt, seed, d=d, F=200, r=16)


def _rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def pin_support_and_ones(O, seed=3):
    """True-support mask == dense == all-ones mask; neurons off the support add exactly 0."""
    for act, wfmt, inp in _identity_cases(seed):
        W = O.Weights(act, wfmt, inp)
        for t in range(inp["x"].shape[0]):
            x = inp["x"][t, 0]
            yd = O.ffn_dense(W, x)
            assert _rel(O.ffn_neurons(W, x, np.arange(W.F)), yd) == 0.0, (act, wfmt, "ones")
            pa = O.preact(W, x)
            key = "g" if act == "reglu" else "a"
            support = np.flatnonzero(pa[key] > 0)
            assert _rel(O.ffn_neurons(W, x, support), yd) < 1e-12, (act, wfmt, "support")
            # complement of the support contributes exactly nothing
            off = np.setdiff1d(np.arange(W.F), support)
            assert np.all(O.ffn_neurons(W, x, off) == 0.0), (act, wfmt, "off-support")


def pin_additivity(O, seed=4):
    rng = np.random.default_rng(seed)
    for act, wfmt, inp in _identity_cases(seed):
        W = O.Weights(act, wfmt, inp)
        x = inp["x"][0, 0]
        perm = rng.permutation(W.F)
        m1, m2 = np.sort(perm[:70]), np.sort(perm[70:150])
        y1, y2 = O.ffn_neurons(W, x, m1), O.ffn_neurons(W, x, m2)
        y12 = O.ffn_neurons(W, x, np.union1d(m1, m2))
        assert _rel(y12, y1 + y2) < 1e-12, (act, wfmt, "additivity")
        # summing every neuron's own contribution gives the dense FFN
        ysum = sum(O.ffn_neurons(W, x, [i]) for i in range(W.F))
        assert _rel(ysum, O.ffn_dense(W, x)) < 1e-12, (act, wfmt, "sum of singletons")


def pin_empty(O):
    for act, wfmt, inp in _identity_cases(5):
        W = O.Weights(act, wfmt, inp)
        y = O.ffn_neurons(W, inp["x"][0, 0], np.array([], dtype=np.int64))
        assert y.shape == (inp["x"].shape[-1],) and np.all(y == 0.0), (act, wfmt, "empty")


# ----------------------------------------------------------------------------- predictor statistics
def pin_rate_closed_form(O, tokens=20000, chunk=4000, seed=11):
    """Empirical firing rate of every neuron (c1 shapes) vs its target p_i, 5-sigma binomial bound."""
    inp = gen.make(configs.C1, ffn=False, tokens=False)
    p = inp["rates"]
    rng = np.random.default_rng(seed)
    hits = np.zeros(configs.C1.F)
    for _ in range(tokens // chunk):
        x = rng.standard_normal((chunk, configs.C1.d))
        lg = O.predictor_logits(x, inp["w_p1"], inp["w_p2"], inp["bias"])
        hits += O.predicted_active(lg, O.logit_threshold(0.5)).sum(axis=0)
    rate = hits / tokens
    bound = 5.0 * np.sqrt(p * (1 - p) / tokens) + 1.0 / tokens
    bad = np.flatnonzero(np.abs(rate - p) > bound)
    assert bad.size == 0, ("rates off the closed form", bad[:10], rate[bad[:10]], p[bad[:10]])
    assert abs(rate.mean() - configs.C1.mean_rate) < 0.003, ("mean rate", rate.mean())


# ----------------------------------------------------------------------------- compaction
def check_compaction(O, active):
    active = np.asarray(active, dtype=bool)
    F = active.shape[-1]
    idx = O.compact(active)
    assert np.all(np.diff(idx) > 0), "ascending and unique"
    assert idx.size == int(active.sum()), "count = popcount"
    assert idx.size == 0 or (idx[0] >= 0 and idx[-1] < F), "in range"
    back = np.zeros(F, bool)
    back[idx] = True
    assert np.array_equal(back, active), "round trip"
    words = O.mask_words(active)
    assert words.shape == ((F + 31) // 32,)
    assert sum(bin(int(w)).count("1") for w in words) == idx.size, "mask popcount"
    for i in idx[:50]:
        assert (int(words[i // 32]) >> (i % 32)) & 1 == 1, "bit position"
    assert np.array_equal(O.words_to_active(words, F), active), "words round trip"


def pin_compaction(O, seed=6):
    rng = np.random.default_rng(seed)
    for F in (1, 31, 32, 33, 1000, 4096):
        for p in (0.0, 0.05, 0.5, 1.0):
            check_compaction(O, rng.random(F) < p)
    masks = rng.random((5, 200)) < 0.1
    u = O.union_active(masks)
    assert np.array_equal(u, np.logical_or.reduce(masks, axis=0)), "union = OR"
    assert np.array_equal(O.compact(u), np.unique(np.concatenate([O.compact(m) for m in masks]))), \
        "union = set union"


def pin_threshold_strict(O):
    lg = np.array([0.0, 1e-300, -1e-300, 5e-5, -5e-5, 2e-4])
    act = O.predicted_active(lg, O.logit_threshold(0.5))
    assert list(act) == [False, True, False, True, False, True], "strict l > 0"
    band = O.exclusion_band(lg, 0.0, 1e-4)
    assert list(band) == [True, True, True, True, True, False], "band |l| < 1e-4"
    assert abs(O.logit_threshold(0.5)) == 0.0
    assert abs(O.logit_threshold(0.75) - math.log(3.0)) < 1e-15


# ----------------------------------------------------------------------------- int4 codec
def pin_int4_roundtrip(O, seed=8):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((64, 512)) * 0.01).astype(np.float32)
    w[3, :128] = 0.0                        # an all-zero group: scale 0, value 0
    packed, scales = gen.quantize_int4_g128(w)
    deq = O.unpack_int4(packed, scales)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    err = np.abs(deq - w.astype(np.float64))
    # RTN: half a step, plus the fp16 rounding of the scale (|q| <= 7 steps of it)
    assert np.all(err <= 0.5 * s + 7 * s * 2.0 ** -11 + 1e-12), "RTN error bound"
    assert np.all(deq[3, :128] == 0.0), "zero group"
    # the largest element of each group lands on q = +-7
    g = w.reshape(64, 4, 128)
    amax = np.abs(g).argmax(axis=2)
    for i in range(0, 64, 7):
        for j in range(4):
            if scales[i, j] == 0:
                continue
            k = j * 128 + amax[i, j]
            assert abs(round(deq[i, k] / float(scales[i, j]))) == 7, "absmax -> |q| = 7"


# ----------------------------------------------------------------------------- one decode step
def pin_token_step(O):
    """token_step composes predict -> strict threshold -> band -> table -> FFN on that table.

    Against the hand-worked example: neurons 3 and 5 sit exactly on the threshold, so they are
    inactive and form the exclusion band; the FFN runs on {0, 2, 4} only.  Against brute force
    on tiny shapes: the table is the set of brute-force logits above 0, the band the set within
    1e-4 of it, and y the brute-force FFN over that table (not the dense FFN).
    """
    ex = _load("worked_example.json")
    inp = {"w_p1": np.array(ex["w_p1"], np.float16), "w_p2": np.array(ex["w_p2"], np.float16),
           "bias": np.array(ex["bias"], np.float32)}
    x = np.array(ex["x"], np.float16)
    for a in ("relu", "reglu"):
        W = O.Weights(a, "f16", _ffn_inputs(ex, a))
        st = O.token_step(inp, W, x)
        assert np.array_equal(st["logits"], np.array(ex["logits"], float)), (a, "step logits")
        assert list(st["idx"]) == ex["active_idx"], (a, "step idx", st["idx"])
        assert list(np.flatnonzero(st["active"])) == ex["active_idx"], (a, "step active")
        assert list(np.flatnonzero(st["band"])) == [3, 5], (a, "step band", st["band"])
        assert np.array_equal(st["y"], np.array(ex[a + "_y_pred"], float)), (a, "step y", st["y"])
    for seed in (1, 2):
        for act, wfmt, d in (("relu", "f16", 8), ("reglu", "f16", 8), ("reglu", "i4g128", 128)):
            inp = _tiny_inputs(act, wfmt, seed, d=d, F=16, r=2)
            W = O.Weights(act, wfmt, inp)
            for t in range(inp["x"].shape[0]):
                x = inp["x"][t, 0]
                bl = _brute_logits(x, inp["w_p1"], inp["w_p2"], inp["bias"])
                st = O.token_step(inp, W, x)
                want = [i for i in range(16) if bl[i] > 0]
                assert list(st["idx"]) == want, (act, wfmt, "step idx", st["idx"], want)
                assert list(np.flatnonzero(st["band"])) == \
                    [i for i in range(16) if abs(bl[i]) < 1e-4], (act, wfmt, "step band")
                yb = _brute_ffn(inp, act, wfmt, x, want, d)
                assert np.allclose(st["y"], yb, rtol=1e-11, atol=1e-12), (act, wfmt, "step y")


ALL_PINS = [pin_worked_example, pin_int4_worked, pin_bruteforce, pin_support_and_ones,
            pin_additivity, pin_empty, pin_rate_closed_form, pin_compaction,
            pin_threshold_strict, pin_int4_roundtrip, pin_token_step]
