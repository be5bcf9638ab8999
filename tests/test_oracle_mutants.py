"""Plant plausible mistakes in the CPU oracle and show that the pins catch each one.

Every mutant below replaces one oracle function (on the CPU, for the duration
of one test) with a version carrying a single mistake of the kind the pins
are meant to stop: a dropped term, a wrong sign or index, a transposed or
swapped operand, an off-by-one, a wrong bit order.  At least one pin must fail
for every mutant.
"""
import numpy as np
import pytest

import oracle.pi_oracle as O

from . import _pins

f64 = O.f64


def _pred_no_bias(x, w_p1, w_p2, bias):
    return (f64(x) @ f64(w_p1)) @ f64(w_p2)


def _pred_minus_bias(x, w_p1, w_p2, bias):
    return (f64(x) @ f64(w_p1)) @ f64(w_p2) - f64(bias)


def _pred_rounded_z(x, w_p1, w_p2, bias):
    z = (f64(x) @ f64(w_p1)).astype(np.float16).astype(np.float64)
    return z @ f64(w_p2) + f64(bias)


def _pred_reversed_bias(x, w_p1, w_p2, bias):
    return (f64(x) @ f64(w_p1)) @ f64(w_p2) + f64(bias)[::-1]


def _active_ge(logits, theta=0.0):
    return f64(logits) >= theta


def _active_sigmoid_wrong(logits, theta=0.0):
    return 1.0 / (1.0 + np.exp(-f64(logits))) > 0.25


def _compact_off_by_one(active):
    return np.flatnonzero(np.asarray(active, bool)) + 1


def _compact_descending(active):
    return np.flatnonzero(np.asarray(active, bool))[::-1]


def _unpack_swapped_nibbles(packed, scales):
    packed = np.asarray(packed, np.uint8)
    rows, half = packed.shape
    u = np.empty((rows, 2 * half), np.int64)
    u[:, 0::2] = packed >> 4
    u[:, 1::2] = packed & 0x0F
    return (u - 8) * np.repeat(f64(scales), 128, axis=1)


def _unpack_offset7(packed, scales):
    packed = np.asarray(packed, np.uint8)
    rows, half = packed.shape
    u = np.empty((rows, 2 * half), np.int64)
    u[:, 0::2] = packed & 0x0F
    u[:, 1::2] = packed >> 4
    return (u - 7) * np.repeat(f64(scales), 128, axis=1)


def _unpack_tiled_scales(packed, scales):
    packed = np.asarray(packed, np.uint8)
    rows, half = packed.shape
    u = np.empty((rows, 2 * half), np.int64)
    u[:, 0::2] = packed & 0x0F
    u[:, 1::2] = packed >> 4
    return (u - 8) * np.tile(f64(scales), (1, 128))


def _ffn_no_relu(W, x, idx):
    xf, idx = f64(x), np.asarray(idx, np.int64)
    a = W.rows("up", idx) @ xf
    h = a if W.act == "relu" else np.maximum(W.rows("gate", idx) @ xf, 0) * a
    return h @ W.rows("down", idx)


def _ffn_gate_up_swapped(W, x, idx):
    xf, idx = f64(x), np.asarray(idx, np.int64)
    a = W.rows("up", idx) @ xf
    if W.act == "relu":
        h = np.maximum(a, 0)
    else:
        h = np.maximum(a, 0) * (W.rows("gate", idx) @ xf)
    return h @ W.rows("down", idx)


def _ffn_down_uses_up(W, x, idx):
    xf, idx = f64(x), np.asarray(idx, np.int64)
    a = W.rows("up", idx) @ xf
    h = np.maximum(a, 0) if W.act == "relu" else np.maximum(W.rows("gate", idx) @ xf, 0) * a
    return h @ W.rows("up", idx)


def _ffn_reglu_relu_both(W, x, idx):
    xf, idx = f64(x), np.asarray(idx, np.int64)
    a = np.maximum(W.rows("up", idx) @ xf, 0)
    h = a if W.act == "relu" else np.maximum(W.rows("gate", idx) @ xf, 0) * a
    return h @ W.rows("down", idx)


def _ffn_drops_last(W, x, idx):
    idx = np.asarray(idx, np.int64)[:-1]
    xf = f64(x)
    a = W.rows("up", idx) @ xf
    h = np.maximum(a, 0) if W.act == "relu" else np.maximum(W.rows("gate", idx) @ xf, 0) * a
    return h @ W.rows("down", idx)


def _ffn_shifted_rows(W, x, idx):
    idx = np.asarray(idx, np.int64)
    xf = f64(x)
    a = W.rows("up", idx) @ xf
    h = np.maximum(a, 0) if W.act == "relu" else np.maximum(W.rows("gate", idx) @ xf, 0) * a
    return h @ W.rows("down", np.minimum(idx + 1, W.F - 1))


def _mask_words_msb_first(active):
    a = np.asarray(active, bool)
    F = a.shape[-1]
    out = np.zeros(a.shape[:-1] + ((F + 31) // 32,), np.uint64)
    for i in range(F):
        out[..., i // 32] |= a[..., i].astype(np.uint64) << np.uint64(31 - i % 32)
    return out.astype(np.uint32)


_token_step_orig = O.token_step


def _step_uses_band(inputs, W, x, theta=0.0, eps=1e-4):
    out = _token_step_orig(inputs, W, x, theta, eps)
    idx = O.compact(out["band"])
    return dict(out, idx=idx, y=O.ffn_neurons(W, x, idx))


def _step_runs_dense(inputs, W, x, theta=0.0, eps=1e-4):
    out = _token_step_orig(inputs, W, x, theta, eps)
    return dict(out, y=O.ffn_dense(W, x))


def _step_mask_or_band(inputs, W, x, theta=0.0, eps=1e-4):
    out = _token_step_orig(inputs, W, x, theta, eps)
    idx = O.compact(out["active"] | out["band"])
    return dict(out, idx=idx, y=O.ffn_neurons(W, x, idx))


def _step_ffn_on_other_token(inputs, W, x, theta=0.0, eps=1e-4):
    out = _token_step_orig(inputs, W, x, theta, eps)
    return dict(out, y=O.ffn_neurons(W, -f64(x), out["idx"]))


MUTANTS = {
    "predictor drops bias": ("predictor_logits", _pred_no_bias),
    "predictor bias sign": ("predictor_logits", _pred_minus_bias),
    "predictor rounds z to fp16": ("predictor_logits", _pred_rounded_z),
    "predictor bias index reversed": ("predictor_logits", _pred_reversed_bias),
    "threshold not strict": ("predicted_active", _active_ge),
    "threshold wrong probability": ("predicted_active", _active_sigmoid_wrong),
    "compaction off by one": ("compact", _compact_off_by_one),
    "compaction descending": ("compact", _compact_descending),
    "int4 nibbles swapped": ("unpack_int4", _unpack_swapped_nibbles),
    "int4 offset 7": ("unpack_int4", _unpack_offset7),
    "int4 scale index k % groups": ("unpack_int4", _unpack_tiled_scales),
    "ffn without relu": ("ffn_neurons", _ffn_no_relu),
    "reglu gate/up swapped": ("ffn_neurons", _ffn_gate_up_swapped),
    "down projection reads up": ("ffn_neurons", _ffn_down_uses_up),
    "reglu clamps up too": ("ffn_neurons", _ffn_reglu_relu_both),
    "ffn drops last neuron": ("ffn_neurons", _ffn_drops_last),
    "down rows shifted": ("ffn_neurons", _ffn_shifted_rows),
    "mask bit order": ("mask_words", _mask_words_msb_first),
    "token_step thresholds the band": ("token_step", _step_uses_band),
    "token_step runs the dense FFN": ("token_step", _step_runs_dense),
    "token_step keeps the band neurons": ("token_step", _step_mask_or_band),
    "token_step FFN on the wrong x": ("token_step", _step_ffn_on_other_token),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in _pins.ALL_PINS:
        try:
            pin(O)
        except (AssertionError, IndexError, ValueError) as e:  # a pin tripped
            failed.append((pin.__name__, str(e)[:80]))
            break                     # one failing pin is enough
    assert failed, f"mutant '{name}' passed every pin"
