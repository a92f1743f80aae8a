"""Gradients of the recurrence (the backward pass for training), fp64.

TEST INFRASTRUCTURE (see the package docstring): the HIP path never uses it.

What is differentiated: the update rule of the dimsnsums.com "GLM-5.3-FLASH"
attention page, section "How can a layer remember without rereading?",

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = S_t^T q_t,

for a loss L with given dL/do_t (dO) and dL/dS_T (dS_T, zero if absent).
The derivation (plain calculus, written out here): with X = Diag(alpha_t)
S_{t-1} and w = v_t - X^T k_t the rule reads S_t = X + beta_t k_t w^T, so
with G = dL/dS_t (everything downstream of S_t, o_t included)

    dv_t     = beta_t G^T k_t
    dbeta_t  = (G^T k_t) . w
    dk_t     = beta_t (G w - X (G^T k_t))
    dq_t     = S_t dO_t
    E        = G - beta_t k_t (G^T k_t)          (= dL/dX)
    dalpha_t = rowsum(E * S_{t-1})               (summed over all entries for
                                                  one rate per head)
    dL/dS_{t-1} = Diag(alpha_t) E  (+ q_{t-1} dO_{t-1}^T from o_{t-1})

and dS0 = dL/dS_0.  The reverse loop below takes these steps from the last
token to the first, re-running the forward recurrence first to have every
S_{t-1}.  Layouts as in recurrence.py; alpha [T, H, d_k] (per key channel)
or [T, H] (one rate per head).
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def kda_backward(q, k, v, alpha, beta, dO, S0=None, dS_T=None, cu_seqlens=None):
    """Returns (dq, dk, dv, dalpha, dbeta, dS0) as float64 arrays shaped like
    q, k, v, alpha, beta and the states [N, H, d_k, d_v]."""
    q, k, v, alpha, beta, dO = map(_f64, (q, k, v, alpha, beta, dO))
    T, H, dk_ = k.shape
    dv_ = v.shape[-1]
    per_head = alpha.shape == (T, H)
    cu = [0, T] if cu_seqlens is None else [int(x) for x in np.asarray(cu_seqlens)]
    N = len(cu) - 1
    out = {name: np.zeros_like(x) for name, x in
           (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha), ("dbeta", beta))}
    dS0 = np.zeros((N, H, dk_, dv_))
    for n in range(N):
        t0, t1 = cu[n], cu[n + 1]
        S = np.zeros((H, dk_, dv_)) if S0 is None else _f64(S0[n]).copy()
        prev = []                                     # S_{t-1} for every token
        for t in range(t0, t1):
            prev.append(S.copy())
            a = alpha[t][:, None] if per_head else alpha[t]        # [H, 1] or [H, d_k]
            X = a[:, :, None] * S
            w = v[t] - np.einsum("hkv,hk->hv", X, k[t])
            S = X + beta[t][:, None, None] * k[t][:, :, None] * w[:, None, :]
        G = np.zeros((H, dk_, dv_)) if dS_T is None else _f64(dS_T[n]).copy()
        for t in range(t1 - 1, t0 - 1, -1):
            Sp = prev[t - t0]
            a = alpha[t][:, None] if per_head else alpha[t]
            b = beta[t][:, None, None]
            X = a[:, :, None] * Sp
            w = v[t] - np.einsum("hkv,hk->hv", X, k[t])
            St = X + b * k[t][:, :, None] * w[:, None, :]
            G = G + q[t][:, :, None] * dO[t][:, None, :]             # o_t = S_t^T q_t
            gk = np.einsum("hkv,hk->hv", G, k[t])                   # G^T k
            out["dv"][t] = beta[t][:, None] * gk
            out["dbeta"][t] = np.einsum("hv,hv->h", gk, w)
            out["dk"][t] = beta[t][:, None] * (np.einsum("hkv,hv->hk", G, w)
                                               - np.einsum("hkv,hv->hk", X, gk))
            out["dq"][t] = np.einsum("hkv,hv->hk", St, dO[t])
            E = G - b * k[t][:, :, None] * gk[:, None, :]
            da = np.sum(E * Sp, axis=2)                              # [H, d_k]
            out["dalpha"][t] = da.sum(axis=1) if per_head else da
            G = a[:, :, None] * E
        dS0[n] = G
    return out["dq"], out["dk"], out["dv"], out["dalpha"], out["dbeta"], dS0
