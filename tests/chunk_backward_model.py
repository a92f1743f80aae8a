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
each chunk's G'.  The decay enters through cumulative log-rates
g = cumsum(log alpha) here, so the model needs alpha > 0 (a kernel would use
products of alpha and exclude alpha_s instead of dividing by it).
"""

from __future__ import annotations

import numpy as np

C = 64


def _masked_decay(g, inclusive):
    """exp(g_r - g_j) per channel for j < r (or j <= r), zero elsewhere:
    [C, C, d]."""
    n = g.shape[0]
    r, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    keep = (j <= r) if inclusive else (j < r)
    diff = np.where(keep[:, :, None], g[:, None, :] - g[None, :, :], -np.inf)
    return np.exp(diff), keep


def _factors(k, q, alpha, beta):
    """The chunk's forward factors from padded k, q, alpha [C, d], beta [C]."""
    g = np.cumsum(np.log(alpha), axis=0)
    Es, strict = _masked_decay(g, inclusive=False)
    Ei, incl = _masked_decay(g, inclusive=True)
    A = np.einsum("rc,jc,rjc->rj", k, k, Es)
    M = np.einsum("rc,jc,rjc->rj", q, k, Ei)
    L = np.eye(C) + beta[:, None] * A
    X = np.linalg.inv(L)
    T = X * beta[None, :]
    Gam = np.exp(g)
    GC = Gam[-1]
    return dict(g=g, Es=Es, Ei=Ei, strict=strict, incl=incl, A=A, M=M, X=X, T=T, Gam=Gam, GC=GC,
                Khat=Gam * k, Qhat=Gam * q, Ktil=(GC[None, :] / Gam) * k)


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
        pa = np.einsum("rj,rc,jc,rjc->rjc", dA, kc, kc, Es)
        dg = pa.sum(axis=1) - pa.sum(axis=0)
        dq = np.einsum("rj,jc,rjc->rc", dM, kc, Ei)
        dk += np.einsum("rj,rc,rjc->jc", dM, qc, Ei)
        pm = np.einsum("rj,rc,jc,rjc->rjc", dM, qc, kc, Ei)
        dg += pm.sum(axis=1) - pm.sum(axis=0)
        # decayed keys and queries, and the chunk's total decay
        Gam, GC = F["Gam"], F["GC"]
        dk += dKhat * Gam
        dg += dKhat * F["Khat"]
        dq += dQhat * Gam
        dg += dQhat * F["Qhat"]
        dk += dKtil * (GC[None, :] / Gam)
        dg -= dKtil * F["Ktil"]
        dg[-1] += np.sum(dKtil * F["Ktil"], axis=0) + dGC * GC
        # g = cumsum(log alpha)
        dlog = np.cumsum(dg[::-1], axis=0)[::-1]
        gq[c0:c0 + n] = dq[:n]
        gk[c0:c0 + n] = dk[:n]
        gv[c0:c0 + n] = dU[:n]
        ga[c0:c0 + n] = (dlog / ac)[:n]
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
