"""Exact-rational KDA checker (fractions.Fraction, pure Python loops).

TEST INFRASTRUCTURE (see the package docstring).

Source: dimsnsums.com "GLM-5.3-FLASH" attention page, section "How can a
layer remember without rereading?", update rule, evaluated in exact rational
arithmetic as the literal product (I - beta k k^T) Diag(alpha_t) S + beta k v^T
with readout o_t = S_t^T q_t.  With dyadic inputs the fp64 oracle must agree
to within its own rounding; this pins that rounding.
"""

from __future__ import annotations

from fractions import Fraction


def _mat(rows, cols, fill=Fraction(0)):
    return [[fill for _ in range(cols)] for _ in range(rows)]


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    C = _mat(n, p)
    for i in range(n):
        for j in range(p):
            acc = Fraction(0)
            for t in range(m):
                acc += A[i][t] * B[t][j]
            C[i][j] = acc
    return C


def kda_exact(q, k, v, alpha, beta, S0=None):
    """Inputs as nested lists (or arrays) of numbers convertible to Fraction.

    q, k, alpha: [T][d_k]; v: [T][d_v]; beta: [T]; S0: [d_k][d_v] or None.
    Returns (o, S_T) as nested lists of Fraction.
    """
    F = Fraction
    T = len(k)
    dk = len(k[0])
    dv = len(v[0])
    S = _mat(dk, dv) if S0 is None else [[F(x) for x in row] for row in S0]
    o = []
    for t in range(T):
        kt = [F(x) for x in k[t]]
        bt = F(beta[t])
        erase = _mat(dk, dk)
        decay = _mat(dk, dk)
        for i in range(dk):
            decay[i][i] = F(alpha[t][i])
            for j in range(dk):
                erase[i][j] = (F(1) if i == j else F(0)) - bt * kt[i] * kt[j]
        write = [[bt * kt[i] * F(v[t][j]) for j in range(dv)] for i in range(dk)]
        S = _matmul(_matmul(erase, decay), S)
        S = [[S[i][j] + write[i][j] for j in range(dv)] for i in range(dk)]
        qt = [F(x) for x in q[t]]
        o.append([sum((qt[i] * S[i][j] for i in range(dk)), F(0)) for j in range(dv)])
    return o, S
