"""fp64 prologue: raw projections -> the recurrence's inputs (test infrastructure; see
the package docstring).

The step just before the recurrence, as the pages describe it:

* Keys are L2-normalised per (token, head) over d_k.  The delta rule's prediction
  only has the right scale for unit keys (step-by-step page, the warning in "How
  Kimi Delta Attention works step by step" and its FAQ "Why does DeltaNet need keys
  to be normalized?"; deep-dive page, "From attention to recurrent state", and its
  "Numerical stability" notes).
* The retention gate comes from the token representation as a sigmoid-like value,
  and the write strength beta is a positive scale (deep-dive page, "From attention
  to recurrent state", the paragraph on how the gate is parameterised).

Readings taken where the pages leave the form open:

* k <- k / sqrt(sum_j k_j^2 + eps) with eps = 1e-6 (the pages give no eps; a zero
  key stays zero instead of dividing by zero).
* beta = sigmoid(b) for a raw logit b: positive and bounded by 1.
* alpha = sigmoid(a) for a raw retention logit a, per key channel (KDA) or per token
  and head (Gated DeltaNet); the recurrence takes g = log(alpha) = -softplus(-a).
* The query is not normalised; it is scaled by ``scale`` in the read step as before.

Each transformation is switched on by one bit of ``flags``; flags = 0 passes the
inputs through.
"""

from __future__ import annotations

import numpy as np

NORM_K = 1       # k is a raw projection: L2-normalise it
BETA_LOGIT = 2   # beta is a logit: beta = sigmoid(beta)
GATE_LOGIT = 4   # g is a retention logit a: g = log(sigmoid(a))
EPS = 1e-6


def l2_normalise(k, eps=EPS):
    """k / sqrt(sum k^2 + eps) over the last axis, in float64."""
    k = np.asarray(k, dtype=np.float64)
    return k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)


def sigmoid(x):
    """1 / (1 + exp(-x)) in float64, without overflow for large |x|."""
    x = np.asarray(x, dtype=np.float64)
    return np.exp(-np.logaddexp(0.0, -x))


def log_sigmoid(x):
    """log(sigmoid(x)) = -softplus(-x) = -log(1 + exp(-x)), in float64."""
    return -np.logaddexp(0.0, -np.asarray(x, dtype=np.float64))


def prologue(k, g, beta, flags):
    """Apply the switched-on transformations; returns (k, g, beta) as float64 (g may
    be None: no decay)."""
    k = np.asarray(k, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    if flags & NORM_K:
        k = l2_normalise(k)
    if flags & BETA_LOGIT:
        beta = sigmoid(beta)
    if g is not None:
        g = np.asarray(g, dtype=np.float64)
        if flags & GATE_LOGIT:
            g = log_sigmoid(g)
    return k, g, beta
