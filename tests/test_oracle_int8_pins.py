"""Pins of the oracle's int8 group-128 dequantizer (the optional int8 predictor): hand-worked
values, the round-to-nearest bound against the generator's quantizer, exact round trips on
the quantization grid, and the transposed layout of the predictor factors.

Format (LLM Runtime page, "Model Quantization": weight-only, per-group scales): W[i, k] =
q[i, k] * s[i, k // 128], q a signed byte, s fp16.
"""
import numpy as np
import pytest

from synth import configs, gen
import oracle.pi_oracle as O


def test_dequant_worked_example():
    q = np.zeros((2, 256), np.int8)
    q[0, :5] = [-127, -1, 0, 1, 127]
    q[0, 128:130] = [3, -3]
    q[1, 255] = -128                                   # the one byte value outside +-127
    s = np.array([[0.25, 2.0], [1.0, 0.5]], np.float16)
    W = O.dequant_int8(q, s)
    assert W.dtype == np.float64 and W.shape == (2, 256)
    assert list(W[0, :5]) == [-31.75, -0.25, 0.0, 0.25, 31.75]
    assert list(W[0, 128:130]) == [6.0, -6.0]
    assert W[1, 255] == -64.0
    assert np.count_nonzero(W) == 7


def test_quantize_dequantize_bound_and_exact_grid():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((16, 384)) * 0.05).astype(np.float16)
    q, s = gen.quantize_int8_g128(w)
    assert q.dtype == np.int8 and s.dtype == np.float16 and s.shape == (16, 3)
    err = np.abs(O.dequant_int8(q, s) - w.astype(np.float64))
    bound = np.repeat(s.astype(np.float64), 128, axis=1) * 0.51
    assert np.all(err <= bound)
    # weights on the grid k * 2^-8 with max |k| = 127 come back exactly
    k = rng.integers(-127, 128, size=(4, 128))
    k[:, 0] = 127
    q2, s2 = gen.quantize_int8_g128((k * 2.0 ** -8).astype(np.float32))
    assert np.all(s2 == np.float16(2.0 ** -8))
    assert np.array_equal(O.dequant_int8(q2, s2), k * 2.0 ** -8)


def test_predictor_from_int8_is_transposed():
    cfg = configs.tiny("relu", "f16", d=256, F=200, r=128, seed=3)
    inp = gen.make(cfg, ffn=False, tokens=False)
    p = gen.predictor_int8(inp)
    W1, W2 = O.predictor_from_int8(p["q_p1t"], p["s_p1t"], p["q_p2t"], p["s_p2t"])
    assert W1.shape == (256, 128) and W2.shape == (128, 200)
    # column j of W_p1 is row j of the transposed factor
    j, kk = 5, 200
    assert W1[kk, j] == float(p["q_p1t"][j, kk]) * float(p["s_p1t"][j, kk // 128])
    assert np.max(np.abs(W2 - inp["w_p2"].astype(np.float64))) <= float(p["s_p2t"].max()) * 0.51
