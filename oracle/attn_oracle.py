"""Plain float64 CPU oracle of the attention side of the layer: its predictor and head-sparse
projections.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or call this module.  The product path never imports it, and it
imports nothing from the product path.

What is computed, and where the pages say so (PowerInfer article, "Adaptive Sparsity
Predictors"): every Transformer layer carries two predictors, one for the neurons of the MLP
block and one for those of the self-attention block, and only the neurons predicted to fire are
computed.  "Neuron-aware Operator": the selected rows and columns are read straight out of the
dense matrices.

Readings where the pages are silent (each listed in the design notes):
* the "neurons" of the self-attention block are its heads: head h owns d_head rows each of W_q,
  W_k and W_v and the matching d_head columns of W_o;
* the attention predictor has the MLP predictor's form, l = (x W_a1) W_a2 + b with one output
  per head, and the same strict test l > 0 (sigmoid(l) > 0.5);
* the projections are stored head-major: w_qkv [H, 3, d_head, d] holds head h's q, k, v rows
  contiguously and w_o [H, d_head, d] holds the rows of W_o^T that head h's output multiplies;
* the attention core over the KV cache is outside this path: the per-head output o [H, d_head]
  arrives as an input, and only the predicted heads' o is read;
* a head predicted inactive gets q = k = v = 0 and contributes nothing to the output.

Every value is computed in float64 from the stored fp16 / fp32 inputs.
"""
from __future__ import annotations

import numpy as np

from .pi_oracle import compact, exclusion_band, f64, predicted_active, predictor_logits


def head_logits(x, w_a1, w_a2, bias_a) -> np.ndarray:
    """Attention predictor logits l [.., H] = (x W_a1) W_a2 + b: the MLP predictor's form with
    one output per head ("Adaptive Sparsity Predictors")."""
    return predictor_logits(x, w_a1, w_a2, bias_a)


def qkv_heads(w_qkv, x, heads) -> np.ndarray:
    """q, k, v of the listed heads, zero for every other head: out [H, 3, d_head] with
    out[h, m, c] = sum_k w_qkv[h, m, c, k] x[k] for h in heads."""
    w = np.asarray(w_qkv)
    H, three, dh, d = w.shape
    out = np.zeros((H, three, dh), np.float64)
    xf = f64(x)
    for h in np.asarray(heads, np.int64):
        out[h] = f64(w[h]).reshape(three * dh, d).dot(xf).reshape(three, dh)
    return out


def qkv_dense(w_qkv, x) -> np.ndarray:
    """q, k, v of every head."""
    return qkv_heads(w_qkv, x, np.arange(np.asarray(w_qkv).shape[0]))


def out_heads(w_o, o, heads) -> np.ndarray:
    """Output projection over the listed heads: y [d] = sum_{h in heads} sum_c o[h, c] w_o[h, c, :]."""
    w = np.asarray(w_o)
    y = np.zeros(w.shape[2], np.float64)
    of = f64(o)
    for h in np.asarray(heads, np.int64):
        y += of[h].dot(f64(w[h]))
    return y


def out_dense(w_o, o) -> np.ndarray:
    """Output projection over every head."""
    return out_heads(w_o, o, np.arange(np.asarray(w_o).shape[0]))


def attn_step(inputs: dict, x, o, theta: float = 0.0, eps: float = 1e-4) -> dict:
    """One token through the attention side: predict the heads, threshold strictly, list the
    active heads in ascending order, project q, k, v of those heads, and project the given
    attention output o [H, d_head] of those heads back to the model width."""
    logits = head_logits(x, inputs["w_a1"], inputs["w_a2"], inputs["bias_a"])
    active = predicted_active(logits, theta)
    heads = compact(active)
    return dict(logits=logits, active=active, band=exclusion_band(logits, theta, eps), heads=heads,
                qkv=qkv_heads(inputs["w_qkv"], x, heads), y=out_heads(inputs["w_o"], o, heads))
