"""A numpy model of a chunked backward pass of the KDA layer, in float64.

This is design groundwork, not the oracle (that is oracle/backward.py, a
token-by-token reverse recurrence).  It differentiates the chunked form the
prefill kernels use -- per 64-token chunk, with S the state at the chunk
start and the chunk's decay, Gram and UT factors

    U = V - Khat S,   W = T U,   O = Qhat S + M W,   S' = Diag(Gamma_C) S + Ktil^T W

-- chunk by chunk in reverse: the state gradient crosses chunks through

    dW = M^T dO + Ktil G',   dU = T^T dW,
    dS = Qhat^T dO + Diag(Gamma_C) G' - Khat^T dU      (G' = dL/dS')

and everything else of a chunk (dq, dk, dv, dalpha, dbeta) comes from
matrix products of that chunk's own quantities, so on a GPU every chunk's
gradients could be formed in parallel once the reverse pass has produced
each chunk's G'.

Every decay factor is a product of rates, E[r, j] = prod_{j < s <= r}
alpha_s (never a quotient), and dalpha_t collects, for every factor that
contains alpha_t, the product of its other rates, through three linear
recurrences per channel (see _decay_grad).  So the model, like the
token-level kernels, is exact when a rate is 0.
"""

from __future__ import annotations

import numpy as np

C = 64


def _range_products(alpha):
    """E[r, j, c] = prod over j < s <= r of alpha[s, c] for j <= r (1 on the
    diagonal), 0 above it: [C, C, d]."""
    n = alpha.shape[0]
    E = np.zeros((n, n, alpha.shape[1]))
    for j in range(n):
        E[j, j] = 1.0
        for r in range(j + 1, n):
            E[r, j] = E[r - 1, j] * alpha[r]
    return E


def _factors(k, q, alpha, beta):
    """The chunk's forward factors from padded k, q, alpha [C, d], beta [C]."""
    Ei = _range_products(alpha)
    idx = np.arange(C)
    incl = idx[None, :] <= idx[:, None]     # [r, j]: j <= r
    strict = idx[None, :] < idx[:, None]
    Es = np.where(strict[:, :, None], Ei, 0.0)
    A = np.einsum("rc,jc,rjc->rj", k, k, Es)
    M = np.einsum("rc,jc,rjc->rj", q, k, Ei)
    L = np.eye(C) + beta[:, None] * A
    X = np.linalg.inv(L)
    T = X * beta[None, :]
    Gam = np.cumprod(alpha, axis=0)          # Gamma_r = prod_{s <= r} alpha_s
    GC = Gam[-1]
    Etail = Ei[-1]                           # [r, c] = prod_{r < s < C} alpha_s
    return dict(Es=Es, Ei=Ei, strict=strict, incl=incl, A=A, M=M, X=X, T=T, Gam=Gam, GC=GC,
                Etail=Etail, Khat=Gam * k, Qhat=Gam * q, Ktil=Etail * k)


def _decay_grad(alpha, F, kc, qc, dKhat, dQhat, dKtil, dGC, dA, dM):
    """dL/dalpha_t [C, d] of one chunk, from the gradients of the factors
    that contain rates:
      Gamma_r (in Khat, Qhat; Gamma_C in the state's decay): the other rates
        of Gamma_r are Gamma_{t-1} E[r, t];
      Etail_r (in Ktil): E[C-1, t] E[t-1, r] for r < t;
      E[r, j] (in A, M): E[r, t] E[t-1, j] for j < t <= r.
    Each sum over the factors runs as a linear recurrence in t."""
    n, d = alpha.shape
    E = F["Ei"]
    one = np.ones(d)
    # Gamma terms: R_t = sum_{r >= t} E[r, t] y_r
    y = dKhat * kc + dQhat * qc
    y[-1] = y[-1] + dGC
    R = np.zeros((n, d))
    R[-1] = y[-1]
    for t in range(n - 2, -1, -1):
        R[t] = y[t] + alpha[t + 1] * R[t + 1]
    before = np.vstack([one, F["Gam"][:-1]])          # Gamma_{t-1}, 1 for t = 0
    out = before * R
    # Ktil terms: P_t = sum_{r < t} E[t-1, r] z_r
    z = dKtil * kc
    P = np.zeros((n, d))
    for t in range(1, n):
        P[t] = alpha[t - 1] * P[t - 1] + z[t - 1] if t > 1 else z[0]
    out += E[-1] * P                                   # E[C-1, t] P_t
    # Gram terms: W_t[j] = sum_{r >= t} E[r, t] V[r, j] (j < t), then
    # D_t = sum_{j < t} E[t-1, j] W_t[j]
    V = (dA[:, :, None] * kc[:, None, :] + dM[:, :, None] * qc[:, None, :]) * kc[None, :, :]
    V = np.where(F["strict"][:, :, None], V, 0.0)
    Wt = np.zeros((n, d))                              # W_t[j] for the current t, all j
    for t in range(n - 1, 0, -1):
        Wt = V[t] + (alpha[t + 1] * Wt if t + 1 < n else 0.0)
        out[t] += np.sum(E[t - 1, :t] * Wt[:t], axis=0)
    return out


def _pad(x, n, fill):
    out = np.full((C,) + x.shape[1:], fill, dtype=np.float64)
    out[:n] = x
    return out


def backward_one(q, k, v, alpha, beta, dO, S0, dST):
    """One sequence and head: q, k, alpha [T, dk]; v, dO [T, dv]; beta [T];
    S0, dST [dk, dv].  Returns (dq, dk, dv, dalpha, dbeta, dS0)."""
    T_len, d = k.shape
    dv_ = v.shape[1]
    # forward: the state at every chunk start and each chunk's U, W
    chunks = []
    S = S0.copy()
    for c0 in range(0, T_len, C):
        n = min(C, T_len - c0)
        kc, qc, vc = _pad(k[c0:c0 + n], n, 0.0), _pad(q[c0:c0 + n], n, 0.0), _pad(v[c0:c0 + n], n, 0.0)
        ac, bc = _pad(alpha[c0:c0 + n], n, 1.0), _pad(beta[c0:c0 + n], n, 0.0)
        F = _factors(kc, qc, ac, bc)
        U = vc - F["Khat"] @ S
        W = F["T"] @ U
        chunks.append((c0, n, kc, qc, ac, bc, F, S, U, W))
        S = F["GC"][:, None] * S + F["Ktil"].T @ W
    gq, gk, gv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    ga, gb = np.zeros_like(alpha), np.zeros_like(beta)
    G = dST.copy() if dST is not None else np.zeros((d, dv_))
    for c0, n, kc, qc, ac, bc, F, S, U, W in reversed(chunks):
        dOc = _pad(dO[c0:c0 + n], n, 0.0)
        # through the outputs and the next chunk's state
        dW = F["M"].T @ dOc + F["Ktil"] @ G
        dM = np.where(F["incl"], dOc @ W.T, 0.0)
        dKtil = W @ G.T
        dGC = np.sum(G * S, axis=1)
        dQhat = dOc @ S.T
        dU = F["T"].T @ dW
        dT = np.where(F["incl"], dW @ U.T, 0.0)
        dS = F["Qhat"].T @ dOc + F["GC"][:, None] * G - F["Khat"].T @ dU
        dKhat = -dU @ S.T
        # T = X Diag(beta), X = L^-1, L = I + Diag(beta) A
        dX = dT * bc[None, :]
        dbeta = np.sum(dT * F["X"], axis=0)
        dL = -F["X"].T @ dX @ F["X"].T
        dA = np.where(F["strict"], bc[:, None] * dL, 0.0)
        dbeta += np.sum(np.where(F["strict"], dL * F["A"], 0.0), axis=1)
        # decayed Gram matrices A (k against k) and M (q against k)
        Es, Ei = F["Es"], F["Ei"]
        dk = np.einsum("rj,jc,rjc->rc", dA, kc, Es) + np.einsum("rj,rc,rjc->jc", dA, kc, Es)
        dq = np.einsum("rj,jc,rjc->rc", dM, kc, Ei)
        dk += np.einsum("rj,rc,rjc->jc", dM, qc, Ei)
        # decayed keys and queries
        dk += dKhat * F["Gam"] + dKtil * F["Etail"]
        dq += dQhat * F["Gam"]
        dalpha = _decay_grad(ac, F, kc, qc, dKhat, dQhat, dKtil, dGC, dA, dM)
        gq[c0:c0 + n] = dq[:n]
        gk[c0:c0 + n] = dk[:n]
        gv[c0:c0 + n] = dU[:n]
        ga[c0:c0 + n] = dalpha[:n]
        gb[c0:c0 + n] = dbeta[:n]
        G = dS
    return gq, gk, gv, ga, gb, G


def chunked_backward(q, k, v, alpha, beta, dO, S0=None, dS_T=None, cu_seqlens=None):
    """Layer layout ([T, H, d] tensors, alpha [T, H, d] or [T, H] for one rate
    per head, states [N, H, d, d]); returns (dq, dk, dv, dalpha, dbeta, dS0)
    like oracle.backward.kda_backward."""
    q, k, v, alpha, beta, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta, dO))
    T, H, d = k.shape
    dv_ = v.shape[-1]
    per_head = alpha.shape == (T, H)
    cu = [0, T] if cu_seqlens is None else [int(x) for x in np.asarray(cu_seqlens)]
    N = len(cu) - 1
    out = [np.zeros_like(x) for x in (q, k, v, alpha, beta)]
    dS0 = np.zeros((N, H, d, dv_))
    for n in range(N):
        a, b = cu[n], cu[n + 1]
        for h in range(H):
            al = alpha[a:b, h]
            if per_head:
                al = np.repeat(al[:, None], d, axis=1)
            s0 = np.zeros((d, dv_)) if S0 is None else np.asarray(S0, dtype=np.float64)[n, h]
            dst = None if dS_T is None else np.asarray(dS_T, dtype=np.float64)[n, h]
            gq, gk, gv, ga, gb, gs = backward_one(q[a:b, h], k[a:b, h], v[a:b, h], al, beta[a:b, h],
                                                  dO[a:b, h], s0, dst)
            out[0][a:b, h], out[1][a:b, h], out[2][a:b, h] = gq, gk, gv
            out[3][a:b, h] = ga.sum(axis=1) if per_head else ga
            out[4][a:b, h] = gb
            dS0[n, h] = gs
    return (*out, dS0)
