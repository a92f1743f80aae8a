"""Scalar-gate (Gated DeltaNet) form of the recurrence, token by token, fp64.

TEST INFRASTRUCTURE (see the package docstring): the HIP path never uses it.

Sources.  The ainewsfeed.tech page "GLM-5.3-Flash Configuration Puts Kimi
and DeepSeek Attention Routes in One Model" names Gated DeltaNet layers as
the linear-attention layers of another hybrid model.  The dimsnsums.com
"GLM-5.3-FLASH" attention page, section "How can a layer remember without
rereading?", gives KDA's update rule and presents one learned decay rate per
key channel as what sets KDA apart.  Reading adopted (the pages print no
formula for Gated DeltaNet): the same delta rule with ONE decay rate per
token and head,

    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
    o_t = S_t^T q_t                                   (post-update read-out),

i.e. KDA's Diag(alpha_t) with every diagonal entry equal.  The product is
evaluated here in its own order -- erase, then scale the erased state, then
write -- which for a scalar alpha_t is the same operator as KDA's printed
decay-then-erase order (a scalar commutes with I - beta k k^T).

Layout (token-major): q, k [T, H, d_k]; v [T, H, d_v]; alpha, beta [T, H];
state [N, H, d_k, d_v]; o [T, H, d_v].  Every input is converted exactly to
float64 before any arithmetic.
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def gdn_step(S, q_t, k_t, v_t, alpha_t, beta_t):
    """One token for a batch of independent heads.

    S [..., d_k, d_v], q_t, k_t [..., d_k], v_t [..., d_v], alpha_t and
    beta_t [...].  Returns (S_t, o_t); S is not modified.
    """
    b = beta_t[..., None, None]
    kcol = k_t[..., :, None]
    recalled = np.einsum("...k,...kv->...v", k_t, S)[..., None, :]   # k^T S_{t-1}
    erased = S - b * kcol * recalled                                  # (I - beta k k^T) S_{t-1}
    S_t = alpha_t[..., None, None] * erased + b * kcol * v_t[..., None, :]
    o_t = np.einsum("...kv,...k->...v", S_t, q_t)                     # S_t^T q_t
    return S_t, o_t


def gdn_recurrent(q, k, v, alpha, beta, S0=None, cu_seqlens=None, num_seqs=None):
    """Prefill over every sequence of a packed batch (scalar gate).

    q, k: [T, H, d_k]; v: [T, H, d_v]; alpha, beta: [T, H].
    S0: [N, H, d_k, d_v] or None (zeros).  cu_seqlens: [N+1] offsets, or
    None for a dense batch of ``num_seqs`` equal-length sequences (default 1).
    Returns (o [T, H, d_v], S_T [N, H, d_k, d_v]) as float64.  Sequences are
    independent; a zero-length sequence returns its S0 unchanged.
    """
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    T, H, dk = k.shape
    dv = v.shape[-1]
    if alpha.shape != (T, H) or beta.shape != (T, H):
        raise ValueError("alpha and beta are [T, H] (one rate per token and head)")
    if cu_seqlens is None:
        n = 1 if num_seqs is None else int(num_seqs)
        if n <= 0 or T % n:
            raise ValueError("dense batch needs T divisible by num_seqs")
        cu = [i * (T // n) for i in range(n + 1)]
    else:
        cu = [int(x) for x in np.asarray(cu_seqlens)]
        if cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
            raise ValueError("cu_seqlens must start at 0, be monotone and end at T")
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    ST = np.zeros((N, H, dk, dv))
    for n in range(N):
        S = np.zeros((H, dk, dv)) if S0 is None else _f64(S0[n]).copy()
        for t in range(cu[n], cu[n + 1]):
            S, o[t] = gdn_step(S, q[t], k[t], v[t], alpha[t], beta[t])
        ST[n] = S
    return o, ST


def gdn_decode_step(q, k, v, alpha, beta, S):
    """One new token for each of N sequences (scalar gate).

    q, k: [N, H, d_k]; v: [N, H, d_v]; alpha, beta: [N, H]; S: [N, H, d_k, d_v].
    Returns (o [N, H, d_v], S_new); the input S is not modified.
    """
    S_new, o = gdn_step(_f64(S), _f64(q), _f64(k), _f64(v), _f64(alpha), _f64(beta))
    return o, S_new
