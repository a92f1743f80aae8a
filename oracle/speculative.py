"""Several new tokens per sequence from a live state, with every intermediate
state kept for rollback (speculative verification), fp64.

TEST INFRASTRUCTURE (see the package docstring): the HIP path never uses it.

Source.  The kongchang.com page "18B Active for Just $0.045: How
GLM-5.3-Flash Beat Claude with Hybrid Attention", section "The Architecture
Stack: How Linear and Sparse Interleave" (the fifth item of its list, one MTP
draft layer for speculative decoding, and the paragraph on speculative
decoding after it) describes
the scheme: a draft proposes several tokens, the target model checks them
in parallel, accepted tokens are kept and the rest are rolled back.  For a
recurrent layer the reading is: run the k proposed tokens of each sequence
from its live state (outputs for all k), keep the state after each token,
and once j tokens are accepted make the state after token j the live state
(j = 0 keeps the old one).  Each token is one step of the update rule on the
dimsnsums.com "GLM-5.3-FLASH" attention page (see recurrence.py).

Layout: tokens of sequence n are rows n*k .. n*k+k-1 of q, k, v, alpha, beta
([N*k, H, ...], the dense-batch layout); S [N, H, d_k, d_v]; the kept states
[N, k, H, d_k, d_v].
"""

from __future__ import annotations

import numpy as np

from .recurrence import kda_step
from .scalar_gate import gdn_step


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def decode_tokens(q, k, v, alpha, beta, S, tokens_per_seq):
    """Returns (o [N*k, H, d_v], states [N, k, H, d_k, d_v]); S is not
    modified.  alpha of beta's shape selects the scalar gate."""
    q, k, v, alpha, beta, S = map(_f64, (q, k, v, alpha, beta, S))
    kk = int(tokens_per_seq)
    N = S.shape[0]
    if q.shape[0] != N * kk:
        raise ValueError("q must hold tokens_per_seq tokens for every sequence")
    step = kda_step if alpha.shape == q.shape else gdn_step
    o = np.zeros(v.shape)
    states = np.zeros((N, kk) + S.shape[1:])
    for n in range(N):
        St = S[n].copy()
        for t in range(kk):
            row = n * kk + t
            St, o[row] = step(St, q[row], k[row], v[row], alpha[row], beta[row])
            states[n, t] = St
    return o, states


def commit(S, states, accepted):
    """The live states after verification: S[n] is replaced by the state
    after token accepted[n] (1-based count of accepted tokens, capped at k);
    accepted[n] <= 0 keeps S[n].  Returns a new array."""
    S = _f64(S).copy()
    kk = states.shape[1]
    for n, j in enumerate(np.asarray(accepted).tolist()):
        j = min(int(j), kk)
        if j >= 1:
            S[n] = states[n, j - 1]
    return S
