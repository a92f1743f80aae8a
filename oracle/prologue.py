"""The gate and normalisation prologue in front of the recurrence, fp64.

TEST INFRASTRUCTURE (see the package docstring): the HIP path never uses it.

Source and reading.  The dimsnsums.com "GLM-5.3-FLASH" attention page,
section "How can a layer remember without rereading?", says each key channel
decays at a learned, data-driven rate and that beta sets the strength of the
update; it does not print how the rates are produced.  The reading adopted is
the parameterisation of the layer's synthetic inputs: from per-token
pre-activations (a, b) and raw q, k,

    alpha = exp(-softplus(a)),   softplus(a) = log(1 + e^a)    (each rate in (0, 1))
    beta  = sigmoid(b) = 1 / (1 + e^-b)                          (strength in (0, 1))
    q <- q / max(||q||_2, 1e-12),  k <- k / max(||k||_2, 1e-12)  (per token and head,
                                                                  over the key channels)

then the recurrence runs on the activated values.  a has alpha's layout (one
value per key channel, or one per head for the scalar gate); b has beta's.
"""

from __future__ import annotations

import numpy as np

from .recurrence import kda_decode_step, kda_recurrent
from .scalar_gate import gdn_decode_step, gdn_recurrent

NORM_EPS = 1e-12


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def decay_from_preact(a):
    """alpha = exp(-softplus(a)), softplus evaluated as log(1 + e^a) without
    overflow (np.logaddexp(0, a))."""
    return np.exp(-np.logaddexp(0.0, _f64(a)))


def strength_from_preact(b):
    """beta = 1 / (1 + e^-b)."""
    b = _f64(b)
    return np.exp(-np.logaddexp(0.0, -b))


def l2_normalise(x):
    """x / max(||x||_2, 1e-12) over the last axis."""
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, NORM_EPS)


def activate(q, k, a, b):
    """(q, k, alpha, beta) the recurrence uses, from raw q, k and the
    pre-activations a, b."""
    return l2_normalise(q), l2_normalise(k), decay_from_preact(a), strength_from_preact(b)


def recurrent_from_preact(q, k, v, a, b, S0=None, cu_seqlens=None, num_seqs=None):
    """Prefill from pre-activations: the per-channel recurrence when a has
    q's shape, the scalar-gate recurrence when it has b's shape."""
    qn, kn, alpha, beta = activate(q, k, a, b)
    run = kda_recurrent if alpha.shape == qn.shape else gdn_recurrent
    return run(qn, kn, v, alpha, beta, S0, cu_seqlens=cu_seqlens, num_seqs=num_seqs)


def decode_step_from_preact(q, k, v, a, b, S):
    qn, kn, alpha, beta = activate(q, k, a, b)
    step = kda_decode_step if alpha.shape == qn.shape else gdn_decode_step
    return step(qn, kn, v, alpha, beta, S)
