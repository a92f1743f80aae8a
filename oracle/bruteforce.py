"""Brute-force KDA checker: the printed matrix product, formed literally.

TEST INFRASTRUCTURE (see the package docstring).

Source: dimsnsums.com "GLM-5.3-FLASH" attention page, section "How can a
layer remember without rereading?", update rule.  Unlike ``recurrence``, this
builds the d_k x d_k matrices (I - beta k k^T) and Diag(alpha_t) and the
outer product beta k v^T and multiplies them in the printed order, so it
checks the operator order and the orientation of S independently of the
distributed form the oracle uses.  Readout o_t = S_t^T q_t (post-update).
One head, one sequence, float64; meant for tiny T and d.
"""

from __future__ import annotations

import numpy as np


def kda_bruteforce(q, k, v, alpha, beta, S0=None):
    """q, k, alpha: [T, d_k]; v: [T, d_v]; beta: [T]; S0: [d_k, d_v] or None.

    Returns (o [T, d_v], S_T [d_k, d_v]).
    """
    q, k, v, alpha, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, alpha, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    eye = np.eye(dk)
    o = np.zeros((T, dv))
    for t in range(T):
        erase = eye - beta[t] * np.outer(k[t], k[t])     # (I - beta k k^T)
        decay = np.diag(alpha[t])                         # Diag(alpha_t)
        write = beta[t] * np.outer(k[t], v[t])            # beta k v^T
        S = erase @ decay @ S + write
        o[t] = S.T @ q[t]
    return o, S
