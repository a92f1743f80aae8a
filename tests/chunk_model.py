"""A numpy model of the chunked algorithm the HIP prefill implements.

This is a design check, not the oracle: it follows the same steps as the
kernels (64-token chunks, 16-token blocks with running products of alpha,
block-factored decayed Gram tiles with a direct fallback for blocks whose
decay underflows, a blocked unit-lower-triangular inverse, and the WY-form
state pass) in float64, so tests can confirm on the CPU that the chunked
algebra reproduces the token-by-token oracle before any GPU code runs.  An
optional ``round_operand`` hook lets a test emulate operand rounding.
"""

from __future__ import annotations

import numpy as np

C = 64
BLK = 16
TINY = 2.0 ** -100


def _ident(x):
    return x


def chunk_local(k, q, alpha, beta, round_operand=_ident):
    """k, q, alpha [64, d]; beta [64] (already padded).  Returns (T, M, flags)."""
    d = k.shape[1]
    bp = np.ones((C, d))
    bs = np.ones((C, d))
    bt = np.ones((4, d))
    flags = np.zeros(4, dtype=bool)
    for b in range(4):
        p = np.ones(d)
        for i in range(BLK):
            p = p * alpha[16 * b + i]
            bp[16 * b + i] = p
        bt[b] = p
        s = np.ones(d)
        for i in range(BLK - 1, -1, -1):
            bs[16 * b + i] = s
            s = s * alpha[16 * b + i]
        flags[b] = not np.all(p >= TINY)
    A = np.zeros((C, C))
    M = np.zeros((C, C))
    for R in range(4):
        rows = slice(16 * R, 16 * R + 16)
        kr = round_operand(k[rows] * bp[rows])
        qr = round_operand(q[rows] * bp[rows])
        for J in range(R + 1):
            cols = slice(16 * J, 16 * J + 16)
            if J == R:
                with np.errstate(divide="ignore"):
                    left = np.where(flags[R], 0.0, 1.0 / bp[cols])
            else:
                left = bs[cols].copy()
                for b in range(J + 1, R):
                    left = left * bt[b]
            kl = round_operand(k[cols] * left)
            A[rows, cols] = kr @ kl.T
            M[rows, cols] = qr @ kl.T
    for b in range(4):
        if not flags[b]:
            continue
        for r in range(16 * b, 16 * b + 16):
            for j in range(16 * b, r + 1):
                f = np.ones(d)
                for s in range(j + 1, r + 1):
                    f = f * alpha[s]
                A[r, j] = np.sum(k[r] * k[j] * f)
                M[r, j] = np.sum(q[r] * k[j] * f)
    A = np.tril(A, -1)
    M = np.tril(M)
    L = np.eye(C) + beta[:, None] * A
    X = np.zeros((C, C))
    for b in range(4):
        blk = slice(16 * b, 16 * b + 16)
        Lb = L[blk, blk]
        Xb = np.zeros((16, 16))
        for jj in range(16):
            x = np.zeros(16)
            for i in range(16):
                x[i] = (1.0 if i == jj else 0.0) - Lb[i, :i] @ x[:i]
            Xb[:, jj] = x
        X[blk, blk] = Xb
    for dist in range(1, 4):
        for J in range(4 - dist):
            I = J + dist
            Y = np.zeros((16, 16))
            for K in range(J, I):
                Y += L[16 * I:16 * I + 16, 16 * K:16 * K + 16] @ X[16 * K:16 * K + 16, 16 * J:16 * J + 16]
            X[16 * I:16 * I + 16, 16 * J:16 * J + 16] = -X[16 * I:16 * I + 16, 16 * I:16 * I + 16] @ Y
    T = X * beta[None, :]
    return T, M, flags


def chunk_state_step(S, k, q, v, alpha, T, M, round_operand=_ident):
    """One chunk of the state pass.  Returns (O [64, dv], S_new)."""
    gam = np.cumprod(alpha, axis=0)                    # Gamma_r (inclusive)
    suf = np.ones_like(alpha)
    for r in range(C - 2, -1, -1):
        suf[r] = suf[r + 1] * alpha[r + 1]             # prod_{s>r} alpha_s
    Khat = round_operand(gam * k)
    Qhat = round_operand(gam * q)
    Ktil = round_operand(suf * k)
    Sr = round_operand(S)
    E = Khat @ Sr
    W = round_operand(T) @ round_operand(v - E)
    Wr = round_operand(W)
    O = Qhat @ Sr + round_operand(M) @ Wr
    S_new = gam[-1][:, None] * S + Ktil.T @ Wr
    return O, S_new


def chunk_products(k, alpha, T, M, round_operand=_ident):
    """The chunk-local products of the re-associated state step:
    P = Ktil^T T (d x 64) and MT = M T (64 x 64, lower triangular), each
    formed from rounded operands and rounded once more as stored."""
    suf = np.ones_like(alpha)
    for r in range(C - 2, -1, -1):
        suf[r] = suf[r + 1] * alpha[r + 1]
    Tr = round_operand(T)
    P = round_operand(round_operand(suf * k).T @ Tr)
    MT = round_operand(round_operand(M) @ Tr)
    return P, MT


def chunk_state_step_reassociated(S, k, q, v, alpha, P, MT, round_operand=_ident):
    """One chunk of the state pass in the re-associated form the kernels use:
    U = V - Khat S, O = Qhat S + (M T) U, S_new = Diag(Gamma_C) S + (Ktil^T T) U
    (W = T U is never formed)."""
    gam = np.cumprod(alpha, axis=0)
    Khat = round_operand(gam * k)
    Qhat = round_operand(gam * q)
    Sr = round_operand(S)
    U = round_operand(v - Khat @ Sr)
    O = Qhat @ Sr + MT @ U
    S_new = gam[-1][:, None] * S + P @ U
    return O, S_new


def chunked_prefill(q, k, v, alpha, beta, S0=None, round_operand=_ident, form="wy"):
    """One head, one sequence: q, k, alpha [T, d], v [T, dv], beta [T].
    ``form`` picks the state step: "wy" (W = T (V - Khat S)) or
    "reassociated" (U = V - Khat S with the products Ktil^T T and M T)."""
    T_len, d = k.shape
    dv = v.shape[1]
    S = np.zeros((d, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T_len, dv))
    for c0 in range(0, T_len, C):
        n = min(C, T_len - c0)
        pad = lambda x, fill: np.concatenate([x[c0:c0 + n], np.full((C - n,) + x.shape[1:], fill)])
        kc, qc, vc = pad(k, 0.0), pad(q, 0.0), pad(v, 0.0)
        ac, bc = pad(alpha, 1.0), pad(beta, 0.0)
        T, M, _ = chunk_local(kc, qc, ac, bc, round_operand)
        if form == "wy":
            O, S = chunk_state_step(S, kc, qc, vc, ac, T, M, round_operand)
        else:
            P, MT = chunk_products(kc, ac, T, M, round_operand)
            O, S = chunk_state_step_reassociated(S, kc, qc, vc, ac, P, MT, round_operand)
        o[c0:c0 + n] = O[:n]
    return o, S
