"""KDA oracle: the gated delta-rule recurrence, token by token, in fp64.

TEST INFRASTRUCTURE (see the package docstring): the HIP path never uses it.

Source: dimsnsums.com "GLM-5.3-FLASH" attention page, section "How can a
layer remember without rereading?", the printed update rule

    S_t = (I - beta_t k_t k_t^T) . Diag(alpha_t) . S_{t-1} + beta_t k_t v_t^T

and the paragraph under it (S_t is the state after token t, I the identity,
beta the update strength, Diag(alpha_t) the per-channel decay rates on a
diagonal).  The same section says each head keeps one 128x128 state that each
arriving token updates once.

Readings where the page is silent (each is listed with its reason in the
design notes):
  * readout o_t = S_t^T q_t with the post-update state and no 1/sqrt(d)
    scale (the page prints only the update; this is the delta-rule
    convention);
  * S is d_k x d_v with rows = key channels: k k^T multiplies S from the
    left and k v^T is d_k x d_v, so Diag(alpha_t) scales key rows and alpha
    has one rate per key channel;
  * operator order is the printed equation's (decay, then erase, then
    write), not the order of the prose sentence that follows it;
  * beta, k, v carry the token index t (only alpha_t has it in print).

Layout (token-major, as the HIP library uses): q, k, alpha [T, H, d_k];
v [T, H, d_v]; beta [T, H]; state [N, H, d_k, d_v]; o [T, H, d_v].  Sequence
n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1.  Every input is converted
exactly to float64 before any arithmetic.
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def kda_step(S, q_t, k_t, v_t, alpha_t, beta_t):
    """One token of the update rule for a batch of independent heads.

    S [..., d_k, d_v] (modified in place and returned), q_t, k_t, alpha_t
    [..., d_k], v_t [..., d_v], beta_t [...].  Returns (S_t, o_t).

    The printed product (I - beta k k^T) Diag(alpha) S + beta k v^T is
    evaluated without forming d_k x d_k matrices: with D = Diag(alpha) S,
      (I - beta k k^T) D + beta k v^T = D + beta k (v - D^T k)^T,
    which is the same expression with the matrix product distributed.
    """
    S *= alpha_t[..., :, None]                       # Diag(alpha_t) S_{t-1}
    e = np.einsum("...k,...kv->...v", k_t, S)          # k_t^T (Diag(alpha_t) S_{t-1})
    S += (beta_t[..., None, None] * k_t[..., :, None]) * (v_t - e)[..., None, :]
    o_t = np.einsum("...k,...kv->...v", q_t, S)        # S_t^T q_t (post-update)
    return S, o_t


def kda_recurrent(q, k, v, alpha, beta, S0=None, cu_seqlens=None, num_seqs=None):
    """Prefill: run the recurrence over every sequence of a packed batch.

    q, k, alpha: [T, H, d_k]; v: [T, H, d_v]; beta: [T, H].
    S0: [N, H, d_k, d_v] or None (zeros).  cu_seqlens: [N+1] offsets, or None
    for a dense batch of ``num_seqs`` equal-length sequences (default 1).
    Returns (o [T, H, d_v], S_T [N, H, d_k, d_v]) as float64.

    Sequences are independent; each starts from its own S0[n] (zeros if S0
    is None) and a zero-length sequence returns S0[n] unchanged.
    """
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    T, H, dk = k.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        n = 1 if num_seqs is None else int(num_seqs)
        if n <= 0 or T % n:
            raise ValueError("dense batch needs T divisible by num_seqs")
        cu = np.arange(n + 1, dtype=np.int64) * (T // n)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
            raise ValueError("cu_seqlens must start at 0, be monotone and end at T")
    N = len(cu) - 1
    o = np.zeros((T, H, dv), dtype=np.float64)
    ST = np.zeros((N, H, dk, dv), dtype=np.float64)
    lens = np.diff(cu)
    # Equal-length sequences are stepped together (vectorised across
    # sequences and heads); ragged batches loop over sequences.
    if N > 0 and np.all(lens == lens[0]):
        L = int(lens[0])
        S = np.zeros((N, H, dk, dv)) if S0 is None else _f64(S0).copy()
        qs, ks = (a.reshape(N, L, H, dk) for a in (q, k))
        vs = v.reshape(N, L, H, dv)
        als = alpha.reshape(N, L, H, dk)
        bs = beta.reshape(N, L, H)
        os_ = o.reshape(N, L, H, dv)
        for t in range(L):
            S, os_[:, t] = kda_step(S, qs[:, t], ks[:, t], vs[:, t], als[:, t], bs[:, t])
        ST[:] = S
        return o, ST
    for s in range(N):
        S = np.zeros((H, dk, dv)) if S0 is None else _f64(S0[s]).copy()
        for t in range(cu[s], cu[s + 1]):
            S, o[t] = kda_step(S, q[t], k[t], v[t], alpha[t], beta[t])
        ST[s] = S
    return o, ST


def kda_decode_step(q, k, v, alpha, beta, S):
    """Decode: one new token for each of N sequences, state advanced once.

    q, k, alpha: [N, H, d_k]; v: [N, H, d_v]; beta: [N, H]; S: [N, H, d_k, d_v].
    Returns (o [N, H, d_v], S_new [N, H, d_k, d_v]) as float64; the input S
    is not modified.  Same rule as one token of ``kda_recurrent``.
    """
    S = _f64(S).copy()
    S, o = kda_step(S, _f64(q), _f64(k), _f64(v), _f64(alpha), _f64(beta))
    return o, S


def rel_l2(x, ref):
    """||x - ref||_2 / ||ref||_2 over the whole array, in float64."""
    x = _f64(x)
    ref = _f64(ref)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
