"""Comparison of the HIP path's outputs with the CPU oracle.

Rules (parity contract):
* index sets: for each token, the symmetric difference between the GPU's
  active set and the oracle's lies inside the oracle's exclusion band
  (|l - theta| < 1e-4, decided on the oracle's fp64 logits); the GPU list is
  strictly ascending, its count equals its length, and the GPU bitmask is
  exactly the bitmask of the GPU list;
* FFN: relative L2 error ||y_gpu - y_ref|| / ||y_ref|| <= 1e-3 per token, with
  y_ref the oracle's FFN over the SAME neuron list the GPU used (so a
  band neuron cannot count twice); a zero reference demands an exactly zero y.
"""
from __future__ import annotations

import numpy as np

import oracle.pi_oracle as O

REL_TOL = 1e-3
BAND = 1e-4


def rel_l2(y, ref) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    if n == 0.0:
        return 0.0 if np.all(y == 0) else float("inf")
    return float(np.linalg.norm(y - ref) / n)


def check_index_set(gpu_idx, gpu_mask_words, ref_logits, F, theta=0.0, ctx=""):
    """Returns the number of band neurons where GPU and oracle differ."""
    gi = np.asarray(gpu_idx, np.int64)
    assert gi.size == 0 or (np.all(np.diff(gi) > 0) and gi[0] >= 0 and gi[-1] < F), \
        f"{ctx}: GPU list not strictly ascending / in range"
    gpu_active = np.zeros(F, bool)
    gpu_active[gi] = True
    words = np.asarray(gpu_mask_words).astype(np.uint32)
    assert np.array_equal(words, O.mask_words(gpu_active)), f"{ctx}: GPU mask != bitmask of GPU list"
    ref_active = O.predicted_active(ref_logits, theta)
    band = O.exclusion_band(ref_logits, theta, BAND)
    diff = gpu_active ^ ref_active
    bad = np.flatnonzero(diff & ~band)
    assert bad.size == 0, (f"{ctx}: {bad.size} neurons differ outside the band, e.g. "
                           f"{bad[:5]} logits {np.asarray(ref_logits)[bad[:5]]}")
    return int(diff.sum())


def check_ffn(y_gpu, W, x, idx, ctx="", tol=REL_TOL) -> float:
    ref = O.ffn_neurons(W, x, idx)
    e = rel_l2(y_gpu, ref)
    assert e <= tol, f"{ctx}: rel-L2 {e:.3e} > {tol}"
    return e
