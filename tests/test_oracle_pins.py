"""Pins for the fp64 oracle: what fixes it other than itself.

Each pin is a function of a single-head runner ``run(q, k, v, alpha, beta,
S0) -> (o, S_T)`` so the same pins can be pointed at deliberately broken
variants of the update (``test_pins_catch_planted_mistakes``): every planted
mistake must fail at least one pin, which shows the pins can tell a right
oracle from a plausible wrong one.

Sources: dimsnsums.com "GLM-5.3-FLASH" attention page, section "How can a
layer remember without rereading?" (update rule, its symbol definitions,
128x128 per-head state, the 71.3 MB figure for 34 layers); the readout
o_t = S_t^T q_t is the convention the oracle fixes.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.signal

import oracle
from oracle import kda_bruteforce, kda_decode_step, kda_exact, kda_recurrent, rel_l2


# ---------------------------------------------------------------- runners

def oracle_run(q, k, v, alpha, beta, S0=None):
    """The oracle on one head, one sequence (shapes [T,d] -> [T,1,d])."""
    o, ST = kda_recurrent(q[:, None], k[:, None], v[:, None], alpha[:, None],
                          np.asarray(beta, dtype=np.float64)[:, None],
                          None if S0 is None else np.asarray(S0)[None, None])
    return o[:, 0], ST[0, 0]


def _mutant(step):
    def run(q, k, v, alpha, beta, S0=None):
        q, k, v, alpha = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha))
        beta = np.asarray(beta, dtype=np.float64)
        T, dk = k.shape
        S = np.zeros((dk, v.shape[1])) if S0 is None else np.array(S0, dtype=np.float64)
        o = np.zeros((T, v.shape[1]))
        for t in range(T):
            S, o[t] = step(S, q[t], k[t], v[t], alpha[t], beta[t], alpha[t - 1] if t else alpha[t])
        return o, S
    return run


def _m_decay_columns(S, q, k, v, a, b, ap):
    D = S * a[None, :]
    S = D + b * np.outer(k, v - k @ D)
    return S, S.T @ q


def _m_pre_update_readout(S, q, k, v, a, b, ap):
    D = a[:, None] * S
    o = D.T @ q
    return D + b * np.outer(k, v - k @ D), o


def _m_prose_order(S, q, k, v, a, b, ap):
    E = S - b * np.outer(k, k @ S)
    S = a[:, None] * E + b * np.outer(k, v)
    return S, S.T @ q


def _m_no_beta_in_erase(S, q, k, v, a, b, ap):
    D = a[:, None] * S
    S = D - np.outer(k, k @ D) + b * np.outer(k, v)
    return S, S.T @ q


def _m_transposed_write(S, q, k, v, a, b, ap):
    D = a[:, None] * S
    S = D - b * np.outer(k, k @ D) + b * np.outer(v, k)
    return S, S.T @ q


def _m_erase_sign(S, q, k, v, a, b, ap):
    D = a[:, None] * S
    S = D + b * np.outer(k, k @ D) + b * np.outer(k, v)
    return S, S.T @ q


def _m_decay_after_write(S, q, k, v, a, b, ap):
    E = S - b * np.outer(k, k @ S) + b * np.outer(k, v)
    S = a[:, None] * E
    return S, S.T @ q


def _m_readout_untransposed(S, q, k, v, a, b, ap):
    D = a[:, None] * S
    S = D + b * np.outer(k, v - k @ D)
    return S, S @ q


def _m_stale_alpha(S, q, k, v, a, b, ap):
    D = ap[:, None] * S
    S = D + b * np.outer(k, v - k @ D)
    return S, S.T @ q


MUTANTS = {
    "decay on value columns": _m_decay_columns,
    "readout before the update": _m_pre_update_readout,
    "erase before decay (prose order)": _m_prose_order,
    "beta dropped from erase": _m_no_beta_in_erase,
    "write v k^T instead of k v^T": _m_transposed_write,
    "erase sign flipped": _m_erase_sign,
    "decay applied after the write": _m_decay_after_write,
    "readout S q instead of S^T q": _m_readout_untransposed,
    "decay of the previous token": _m_stale_alpha,
}


# ------------------------------------------------------------ input helpers

def _rand(rng, T, dk, dv, unit_k=True, decay=(0.3, 1.0)):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        q /= np.linalg.norm(q, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    alpha = rng.uniform(decay[0], decay[1], (T, dk))
    beta = rng.uniform(0.05, 1.0, T)
    S0 = rng.standard_normal((dk, dv))
    return q, k, v, alpha, beta, S0


def _dyadic(rng, shape, bits=3, lo=-4, hi=4):
    return rng.integers(lo * 2**bits, hi * 2**bits + 1, shape) / 2.0**bits


# -------------------------------------------------------------------- pins

def pin_golden(run, golden=None):
    """Hand-worked two-token example with d_k=2, d_v=3 (dyadic: exact)."""
    g = golden or _golden()
    o, ST = run(np.array(g["q"], float), np.array(g["k"], float), np.array(g["v"], float),
                np.array(g["alpha"], float), np.array(g["beta"], float), np.array(g["S0"], float))
    assert np.array_equal(o, np.array(g["o"], float)), o
    assert np.array_equal(ST, np.array(g["S_T"], float)), ST


def pin_identity(run):
    """alpha = 1, beta = 0: the state never changes and o_t = S0^T q_t."""
    rng = np.random.default_rng(11)
    q, k, v, _, _, S0 = _rand(rng, 9, 5, 3)
    o, ST = run(q, k, v, np.ones((9, 5)), np.zeros(9), S0)
    assert np.array_equal(ST, S0)                       # bit-exact: x*1 + 0 = x
    assert np.allclose(o, q @ S0, rtol=1e-15, atol=1e-15)


def pin_overwrite(run):
    """alpha = 1, beta = 1, ||k|| = 1: k_t^T S_t = v_t, so with q = k, o_t = v_t."""
    rng = np.random.default_rng(12)
    _, k, v, _, _, S0 = _rand(rng, 7, 6, 4)
    o, _ = run(k, k, v, np.ones((7, 6)), np.ones(7), S0)
    assert np.max(np.abs(o - v)) < 1e-12, np.max(np.abs(o - v))


def pin_beta0_closed_form(run):
    """beta = 0: S_t = Diag(prod_{s<=t} alpha_s) S0 and o_t = S_t^T q_t."""
    rng = np.random.default_rng(13)
    q, k, v, alpha, _, S0 = _rand(rng, 8, 4, 3)
    o, ST = run(q, k, v, alpha, np.zeros(8), S0)
    cum = np.cumprod(alpha, axis=0)
    assert np.allclose(ST, cum[-1][:, None] * S0, rtol=1e-14, atol=1e-15)
    ref_o = np.stack([(cum[t][:, None] * S0).T @ q[t] for t in range(8)])
    assert np.allclose(o, ref_o, rtol=1e-13, atol=1e-15)


def pin_alpha0_erases_history(run):
    """alpha_t = 0 at token t: S_t = beta_t k_t v_t^T whatever came before."""
    rng = np.random.default_rng(14)
    q, k, v, alpha, beta, S0 = _rand(rng, 6, 4, 5)
    alpha[3] = 0.0
    _, ST = run(q[:4], k[:4], v[:4], alpha[:4], beta[:4], S0)
    assert np.allclose(ST, beta[3] * np.outer(k[3], v[3]), rtol=0, atol=1e-15)


def pin_scalar_iir(run):
    """d_k = d_v = 1, constant alpha, beta, k: s_t = (1 - beta k^2) alpha s_{t-1} + beta k v_t,
    a first-order IIR filter; compared with scipy.signal.lfilter."""
    rng = np.random.default_rng(15)
    T = 50
    a, b, kk, qq = 0.9, 0.4, 0.8, 1.3
    v = rng.standard_normal((T, 1))
    o, ST = run(np.full((T, 1), qq), np.full((T, 1), kk), v, np.full((T, 1), a), np.full(T, b), None)
    s = scipy.signal.lfilter([b * kk], [1.0, -(1.0 - b * kk * kk) * a], v[:, 0])
    assert np.allclose(o[:, 0], qq * s, rtol=1e-12, atol=1e-14)
    assert abs(ST[0, 0] - s[-1]) < 1e-12


def pin_lms_gradient_step(run):
    """alpha = 1: one token is one gradient step of size beta on
    L(S) = 1/2 ||S^T k - v||^2 (the delta rule as Widrow-Hoff LMS).  The
    gradient is taken by central finite differences, which are exact up to
    rounding for a quadratic loss."""
    rng = np.random.default_rng(16)
    dk, dv = 4, 3
    q, k, v, _, beta, S0 = _rand(rng, 1, dk, dv)

    def loss(S):
        r = S.T @ k[0] - v[0]
        return 0.5 * float(r @ r)

    h = 1e-3
    grad = np.zeros((dk, dv))
    for i in range(dk):
        for j in range(dv):
            E = np.zeros((dk, dv))
            E[i, j] = h
            grad[i, j] = (loss(S0 + E) - loss(S0 - E)) / (2 * h)
    _, ST = run(q, k, v, np.ones((1, dk)), beta, S0)
    assert np.allclose(ST, S0 - beta[0] * grad, rtol=1e-8, atol=1e-9)


def pin_bruteforce(run):
    """Agreement with the printed matrix product formed literally."""
    rng = np.random.default_rng(17)
    q, k, v, alpha, beta, S0 = _rand(rng, 12, 5, 3, unit_k=False)
    o, ST = run(q, k, v, alpha, beta, S0)
    ob, Sb = kda_bruteforce(q, k, v, alpha, beta, S0)
    assert rel_l2(o, ob) < 1e-13 and rel_l2(ST, Sb) < 1e-13


def pin_exact_rational(run):
    """Agreement with exact rational arithmetic on dyadic inputs."""
    rng = np.random.default_rng(18)
    T, dk, dv = 5, 3, 4
    q, k, v = _dyadic(rng, (T, dk)), _dyadic(rng, (T, dk), lo=-1, hi=1), _dyadic(rng, (T, dv))
    alpha = rng.integers(0, 9, (T, dk)) / 8.0
    beta = rng.integers(0, 9, T) / 8.0
    S0 = _dyadic(rng, (dk, dv))
    o, ST = run(q, k, v, alpha, beta, S0)
    oe, Se = kda_exact(q.tolist(), k.tolist(), v.tolist(), alpha.tolist(), beta.tolist(), S0.tolist())
    oe = np.array([[float(x) for x in r] for r in oe])
    Se = np.array([[float(x) for x in r] for r in Se])
    scale = max(1.0, float(np.max(np.abs(oe))), float(np.max(np.abs(Se))))
    assert np.max(np.abs(o - oe)) <= 1e-13 * scale
    assert np.max(np.abs(ST - Se)) <= 1e-13 * scale


PINS = [pin_golden, pin_identity, pin_overwrite, pin_beta0_closed_form,
        pin_alpha0_erases_history, pin_scalar_iir, pin_lms_gradient_step,
        pin_bruteforce, pin_exact_rational]


def _golden():
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    with open(os.path.join(here, "hand_example_dk2_dv3.json")) as f:
        return json.load(f)


# ------------------------------------------------------------------- tests

@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle_run)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    run = _mutant(MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            pin(run)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"


def test_mutant_runner_matches_oracle_when_unbroken():
    """The harness used for mutants reproduces the oracle with the right step."""
    def right(S, q, k, v, a, b, ap):
        D = a[:, None] * S
        S = D + b * np.outer(k, v - k @ D)
        return S, S.T @ q
    for pin in PINS:
        pin(_mutant(right))


def test_checkers_reproduce_golden():
    """The brute-force and exact-rational checkers are themselves pinned by the
    hand-worked example."""
    g = _golden()
    ob, Sb = kda_bruteforce(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"])
    assert np.array_equal(ob, np.array(g["o"], float)) and np.array_equal(Sb, np.array(g["S_T"], float))
    oe, Se = kda_exact(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["S0"])
    assert [[Fraction(x) for x in r] for r in g["o"]] == oe
    assert [[Fraction(x) for x in r] for r in g["S_T"]] == Se


def test_prose_order_does_not_match():
    """Negative pin: erasing with the undecayed state and decaying afterwards
    (the order of the sentence after the equation) is a different rule; the
    oracle follows the equation and differs from it at the 1e-2 level."""
    g = _golden()
    _, ST = oracle_run(np.array(g["q"], float), np.array(g["k"], float), np.array(g["v"], float),
                       np.array(g["alpha"], float), np.array(g["beta"], float), np.array(g["S0"], float))
    assert not np.allclose(ST, np.array(g["S_T_prose_order"]))
    rng = np.random.default_rng(0)
    q, k, v, alpha, beta, S0 = _rand(rng, 200, 16, 12)
    o1, S1 = oracle_run(q, k, v, alpha, beta, S0)
    o2, S2 = _mutant(_m_prose_order)(q, k, v, alpha, beta, S0)
    assert rel_l2(S2, S1) > 1e-2


def test_state_size_matches_printed_figure(golden_dir):
    """34 layers x 32 heads x 128x128 fp32 = 71,303,168 B, printed as 71.3 MB;
    and the oracle's state for one layer has that per-head shape."""
    with open(os.path.join(golden_dir, "state_size.json")) as f:
        g = json.load(f)
    per_head = g["d_k"] * g["d_v"] * g["bytes_per_element"]
    total = g["kda_layers"] * g["heads_per_layer"] * per_head
    assert total == 71_303_168
    assert round(total / 1e6, 1) == g["printed_megabytes"]
    H, d = g["heads_per_layer"], g["d_k"]
    rng = np.random.default_rng(1)
    T = 3
    x = rng.standard_normal((T, H, d))
    _, ST = kda_recurrent(x, x, x, np.full((T, H, d), 0.5), np.full((T, H), 0.5))
    assert ST.shape == (1, H, d, d)
    assert ST.astype(np.float32).nbytes * g["kda_layers"] == total
