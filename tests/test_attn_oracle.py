"""The attention-side oracle against its pins, and plausible mistakes planted in it caught by
at least one pin (CPU only)."""
import numpy as np
import pytest

import oracle.attn_oracle as A

from . import _pins_attn

f64 = A.f64


@pytest.mark.parametrize("pin", _pins_attn.ALL_PINS, ids=lambda p: p.__name__)
def test_attn_oracle_pin(pin):
    pin(A)


def _logits_no_bias(x, w_a1, w_a2, bias_a):
    return (f64(x) @ f64(w_a1)) @ f64(w_a2)


def _logits_transposed_second(x, w_a1, w_a2, bias_a):
    z = f64(x) @ f64(w_a1)
    w2 = f64(w_a2)
    return (z @ w2[:, ::-1]) + f64(bias_a)


def _dense_qkv(w_qkv, x):
    w = np.asarray(w_qkv)
    H, three, dh, d = w.shape
    return np.stack([f64(w[h]).reshape(three * dh, d).dot(f64(x)).reshape(three, dh) for h in range(H)])


def _qkv_swapped_kv(w_qkv, x, heads):
    out = _ORIG["qkv_heads"](w_qkv, x, heads)
    return out[:, [0, 2, 1], :]


def _qkv_head_off_by_one(w_qkv, x, heads):
    w = np.asarray(w_qkv)
    H, three, dh, d = w.shape
    out = np.zeros((H, three, dh))
    for h in np.asarray(heads, np.int64):
        out[h] = f64(w[(h + 1) % H]).reshape(three * dh, d).dot(f64(x)).reshape(three, dh)
    return out


def _out_all_heads(w_o, o, heads):
    return _ORIG["out_heads"](w_o, o, np.arange(np.asarray(w_o).shape[0]))


def _out_reversed_within_head(w_o, o, heads):
    of = f64(o)[:, ::-1]
    return _ORIG["out_heads"](w_o, of, heads)


def _out_o_of_next_head(w_o, o, heads):
    of = np.roll(f64(o), 1, axis=0)
    return _ORIG["out_heads"](w_o, of, heads)


def _step_threshold_ge(inputs, x, o, theta=0.0, eps=1e-4):
    logits = A.head_logits(x, inputs["w_a1"], inputs["w_a2"], inputs["bias_a"])
    heads = np.flatnonzero(logits >= theta)
    return dict(logits=logits, active=logits >= theta, band=np.abs(logits - theta) < eps, heads=heads,
                qkv=A.qkv_heads(inputs["w_qkv"], x, heads), y=A.out_heads(inputs["w_o"], o, heads))


def _step_descending(inputs, x, o, theta=0.0, eps=1e-4):
    st = _ORIG["attn_step"](inputs, x, o, theta, eps)
    st["heads"] = st["heads"][::-1]
    return st


_ORIG = {n: getattr(A, n) for n in ("head_logits", "qkv_heads", "out_heads", "attn_step")}

MUTANTS = [
    ("head_logits", _logits_no_bias),
    ("head_logits", _logits_transposed_second),
    ("qkv_heads", lambda w, x, heads: _dense_qkv(w, x)),          # ignores the head list
    ("qkv_heads", _qkv_swapped_kv),
    ("qkv_heads", _qkv_head_off_by_one),
    ("out_heads", _out_all_heads),
    ("out_heads", _out_reversed_within_head),
    ("out_heads", _out_o_of_next_head),
    ("attn_step", _step_threshold_ge),
    ("attn_step", _step_descending),
]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=lambda m: getattr(m, "__name__", str(m)))
def test_attn_mutant_caught(monkeypatch, name, fn):
    monkeypatch.setattr(A, name, fn)
    for pin in _pins_attn.ALL_PINS:
        try:
            pin(A)
        except (AssertionError, ValueError, IndexError):
            return
    pytest.fail(f"no pin caught the mutant {fn.__name__} of {name}")
