"""Plain float64 CPU oracle of the predictor-gated, neuron-aware sparse FFN.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module.  The product
path (the HIP library and its Python binding) never imports it, and it
imports nothing from the product path: inputs come from ``synth`` (seeded
draws only) and are handed over as NumPy arrays.

What is computed, and where the pages say so (PowerInfer article, English
spun copy and its Japanese translation):

* Online engine / "Adaptive Sparsity Predictors": for every token a small
  per-layer predictor decides which FFN neurons will fire, and only those
  are computed; the rest are skipped.
* "Neuron Placement and Management": a table maps each kept neuron back to
  its position in the original weight matrix -- here the ascending list of
  predicted-active neuron ids.
* "Neuron-aware Operator": the operator reads the selected neurons' row
  vectors (up / gate projection) and column vectors (down projection)
  straight out of the one dense matrix, with no conversion to a sparse
  format.  Storing the down projection neuron-major makes each neuron's
  output vector one contiguous row.
* Intel Extension for Transformers LLM Runtime, "01 LLM Runtime" and
  "04 Accuracy": weight-only int4 with per-group scales (group 32 or 128)
  produced by round-to-nearest; the same per-group weight-only scheme at 8 bits
  stores the optional int8 predictor.

Readings where the pages are silent (each listed in the design notes):
predictor = linear low-rank pair l = (x W_p1) W_p2 + b with no hidden
nonlinearity; "sigmoid(l) > 0.5" is the strict test l > 0; the index list is
ascending; ReGLU is h = max(x.W_gate, 0) * (x.W_up); int4 is symmetric with
q = u - 8 for the stored nibble u and the even column in the low nibble; each
token of a batch uses its own mask (the batch union is only a schedule).

Every value is computed in float64 from the stored fp16 / int4 / fp32 inputs,
with no blocking, fusion or reordering beyond the definitions.
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 128


def f64(a) -> np.ndarray:
    return np.asarray(a).astype(np.float64)


# ---------------------------------------------------------------------------
# int4 group-128 weights (LLM Runtime page, "01 LLM Runtime": per-group scales)
# ---------------------------------------------------------------------------
def unpack_int4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Dequantise rows of packed int4: W[i, k] = (u[i, k] - 8) * s[i, k // 128].

    packed: uint8 [rows, d/2], byte j holds column 2j in its low nibble and
    column 2j+1 in its high nibble.  scales: fp16 [rows, d/128].
    """
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    d = 2 * half
    u = np.empty((rows, d), dtype=np.int64)
    u[:, 0::2] = packed & 0x0F
    u[:, 1::2] = packed >> 4
    q = (u - 8).astype(np.float64)
    s = np.repeat(f64(scales), GROUP, axis=1)
    assert s.shape == q.shape, "scale count must be d / 128"
    return q * s


# ---------------------------------------------------------------------------
# int8 group-128 predictor factors (LLM Runtime page, "Model Quantization": weight-only
# per-group quantization, here at 8 bits)
# ---------------------------------------------------------------------------
def dequant_int8(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Dequantise rows of int8: W[i, k] = q[i, k] * s[i, k // 128], q the stored signed
    byte.  q: int8 [rows, cols]; scales: fp16 [rows, cols/128]."""
    q = np.asarray(q, dtype=np.int8).astype(np.float64)
    s = np.repeat(f64(scales), GROUP, axis=1)
    assert s.shape == q.shape, "scale count must be cols / 128"
    return q * s


def predictor_from_int8(q_p1t, s_p1t, q_p2t, s_p2t):
    """The fp64 factors (W_p1 [d, r], W_p2 [r, F]) of a predictor stored transposed in
    int8 group-128: the same predictor_logits then applies."""
    return dequant_int8(q_p1t, s_p1t).T, dequant_int8(q_p2t, s_p2t).T


# ---------------------------------------------------------------------------
# Predictor and mask (PowerInfer, "Adaptive Sparsity Predictors" / online engine)
# ---------------------------------------------------------------------------
def logit_threshold(tau: float = 0.5) -> float:
    """sigmoid(l) > tau  <=>  l > ln(tau / (1 - tau)); 0 for tau = 0.5."""
    return math.log(tau / (1.0 - tau))


def predictor_logits(x, w_p1, w_p2, bias) -> np.ndarray:
    """l = (x W_p1) W_p2 + b for x of shape [..., d]; z = x W_p1 is kept unrounded."""
    z = f64(x) @ f64(w_p1)
    return z @ f64(w_p2) + f64(bias)


def predicted_active(logits, theta: float = 0.0) -> np.ndarray:
    """Neuron i is predicted active when its logit exceeds theta (strict)."""
    return f64(logits) > theta


def exclusion_band(logits, theta: float = 0.0, eps: float = 1e-4) -> np.ndarray:
    """Neurons whose logit lies within eps of the threshold: their decision depends on
    rounding order, so index-set comparisons ignore them."""
    return np.abs(f64(logits) - theta) < eps


# ---------------------------------------------------------------------------
# Neuron table (PowerInfer, "Neuron Placement and Management")
# ---------------------------------------------------------------------------
def compact(active) -> np.ndarray:
    """Ascending original positions of the active neurons (int64)."""
    return np.flatnonzero(np.asarray(active, dtype=bool))


def union_active(actives) -> np.ndarray:
    """OR of per-token masks [B, F] -> [F]."""
    return np.asarray(actives, dtype=bool).any(axis=0)


def mask_words(active) -> np.ndarray:
    """Bitmask of an [..., F] boolean array: bit (i % 32) of word (i // 32) is neuron i."""
    a = np.asarray(active, dtype=bool)
    F = a.shape[-1]
    W = (F + 31) // 32
    out = np.zeros(a.shape[:-1] + (W,), dtype=np.uint64)
    for i in range(F):
        out[..., i // 32] |= a[..., i].astype(np.uint64) << np.uint64(i % 32)
    return out.astype(np.uint32)


def words_to_active(words, F: int) -> np.ndarray:
    """Inverse of mask_words."""
    w = np.asarray(words, dtype=np.uint64)
    i = np.arange(F)
    return ((w[..., i // 32] >> (i % 32).astype(np.uint64)) & np.uint64(1)).astype(bool)


# ---------------------------------------------------------------------------
# Neuron-aware FFN (PowerInfer, "Neuron-aware Operator")
# ---------------------------------------------------------------------------
class Weights:
    """The stored FFN matrices of one layer, all neuron-major [F, d].

    fp16: arrays w_up, w_down (and w_gate for ReGLU).  int4: q_* packed uint8
    [F, d/2] with s_* fp16 [F, d/128].  ``rows(name, idx)`` gathers the listed
    neurons' rows and widens them to float64 (dequantising int4).
    """

    def __init__(self, act: str, wfmt: str, arrays: dict):
        if act not in ("relu", "reglu") or wfmt not in ("f16", "i4g128"):
            raise ValueError((act, wfmt))
        self.act, self.wfmt, self.a = act, wfmt, arrays

    @classmethod
    def from_inputs(cls, inputs: dict) -> "Weights":
        cfg = inputs["cfg"]
        return cls(cfg.act, cfg.wfmt, inputs)

    @property
    def F(self) -> int:
        key = "w_up" if self.wfmt == "f16" else "q_up"
        return self.a[key].shape[0]

    def rows(self, name: str, idx) -> np.ndarray:
        idx = np.asarray(idx, dtype=np.int64)
        if self.wfmt == "f16":
            return f64(self.a["w_" + name][idx])
        return unpack_int4(self.a["q_" + name][idx], self.a["s_" + name][idx])


def ffn_neurons(W: Weights, x, idx) -> np.ndarray:
    """y = sum over k of h_k * W_down[i_k, :] for the listed neurons i_k only.

    ReLU:  h_k = max(W_up[i_k] . x, 0)
    ReGLU: h_k = max(W_gate[i_k] . x, 0) * (W_up[i_k] . x)
    An empty list gives y = 0 exactly.
    """
    xf = f64(x)
    idx = np.asarray(idx, dtype=np.int64)
    a = W.rows("up", idx) @ xf
    if W.act == "relu":
        h = np.maximum(a, 0.0)
    else:
        g = W.rows("gate", idx) @ xf
        h = np.maximum(g, 0.0) * a
    return h @ W.rows("down", idx)


def ffn_dense(W: Weights, x) -> np.ndarray:
    """The FFN over all F neurons (no skipping)."""
    return ffn_neurons(W, x, np.arange(W.F))


def preact(W: Weights, x) -> dict:
    """Dense pre-activations a = W_up x (and g = W_gate x) of every neuron."""
    xf = f64(x)
    out = {"a": W.rows("up", np.arange(W.F)) @ xf}
    if W.act == "reglu":
        out["g"] = W.rows("gate", np.arange(W.F)) @ xf
    return out


# ---------------------------------------------------------------------------
# One decode step
# ---------------------------------------------------------------------------
def token_step(inputs: dict, W: Weights, x, theta: float = 0.0, eps: float = 1e-4) -> dict:
    """Predict, threshold, compact and run the sparse FFN for one token x [d]."""
    logits = predictor_logits(x, inputs["w_p1"], inputs["w_p2"], inputs["bias"])
    active = predicted_active(logits, theta)
    idx = compact(active)
    return dict(logits=logits, active=active, band=exclusion_band(logits, theta, eps),
                idx=idx, y=ffn_neurons(W, x, idx))
