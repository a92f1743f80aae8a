"""Pins for the scalar-gate (Gated DeltaNet) oracle, oracle/scalar_gate.py.

What fixes it other than itself:
  * it agrees with the per-channel oracle (written independently, in the
    printed decay-then-erase order, and pinned on its own) when every key
    channel gets the same rate;
  * key-space rotation invariance, which holds for a scalar gate and fails
    for a per-channel one: rotating q, k and the rows of S0 by an orthogonal
    R leaves o unchanged and rotates S_T;
  * closed forms: beta = 0 gives S_t = (prod alpha) S0; alpha_t = 0 erases
    the history, S_t = beta_t k_t v_t^T; d_k = d_v = 1 with constant alpha,
    beta, k is the first-order filter s_t = alpha (1 - beta k^2) s_{t-1}
    + beta k v_t (scipy.signal.lfilter);
  * alpha = 1: one Widrow-Hoff step on 0.5 ||S^T k - v||^2 with step beta;
and every planted mistake below fails at least one of them.
"""

import numpy as np
import pytest
import scipy.signal

from oracle import gdn_decode_step, gdn_recurrent, gdn_step, kda_recurrent


def _inputs(seed, T, H, dk, dv, unit=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    alpha = rng.uniform(0.5, 1.0, (T, H))
    beta = rng.uniform(0.0, 1.0, (T, H))
    return q, k, v, alpha, beta


def _close(a, b, tol=1e-12):
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) <= tol * max(1.0, np.max(np.abs(b)))


# ----------------------------------------------------------------- runners
# A runner maps (q, k, v, alpha, beta, S0, cu) -> (o, S_T); the pins take a
# runner so that the planted mistakes below go through the same checks.

def oracle_runner(q, k, v, alpha, beta, S0=None, cu=None):
    return gdn_recurrent(q, k, v, alpha, beta, S0, cu_seqlens=cu)


def _mutant(step):
    def run(q, k, v, alpha, beta, S0=None, cu=None):
        T, H, dk = q.shape
        dv = v.shape[-1]
        cu = [0, T] if cu is None else list(cu)
        o = np.zeros((T, H, dv))
        ST = np.zeros((len(cu) - 1, H, dk, dv))
        for n in range(len(cu) - 1):
            S = np.zeros((H, dk, dv)) if S0 is None else np.array(S0[n], dtype=np.float64)
            for t in range(cu[n], cu[n + 1]):
                S, o[t] = step(S, q[t], k[t], v[t], alpha[t], beta[t])
            ST[n] = S
        return o, ST
    return run


def _outer(a, b):
    return a[..., :, None] * b[..., None, :]


def _decay_after_write(S, q, k, v, a, b):        # alpha also scales the new write
    kS = np.einsum("hk,hkv->hv", k, S)
    S = a[:, None, None] * (S - b[:, None, None] * _outer(k, kS) + b[:, None, None] * _outer(k, v))
    return S, np.einsum("hkv,hk->hv", S, q)


def _pre_update_readout(S, q, k, v, a, b):       # o_t from S_{t-1}
    o = np.einsum("hkv,hk->hv", a[:, None, None] * S, q)
    kS = np.einsum("hk,hkv->hv", k, S)
    S = a[:, None, None] * (S - b[:, None, None] * _outer(k, kS)) + b[:, None, None] * _outer(k, v)
    return S, o


def _erase_sign(S, q, k, v, a, b):               # + instead of - in the erase
    kS = np.einsum("hk,hkv->hv", k, S)
    S = a[:, None, None] * (S + b[:, None, None] * _outer(k, kS)) + b[:, None, None] * _outer(k, v)
    return S, np.einsum("hkv,hk->hv", S, q)


def _transposed_state(S, q, k, v, a, b):         # erase acts on value columns
    Sk = np.einsum("hkv,hv->hk", S, k[:, : S.shape[2]]) if S.shape[1] == S.shape[2] else None
    S = a[:, None, None] * (S - b[:, None, None] * _outer(Sk, k)) + b[:, None, None] * _outer(k, v)
    return S, np.einsum("hkv,hk->hv", S, q)


def _no_decay_on_erase(S, q, k, v, a, b):        # decay the state, erase with the undecayed recall
    kS = np.einsum("hk,hkv->hv", k, S)
    S = a[:, None, None] * S - b[:, None, None] * _outer(k, kS) + b[:, None, None] * _outer(k, v)
    return S, np.einsum("hkv,hk->hv", S, q)


MUTANTS = {
    "decay_after_write": _decay_after_write,
    "pre_update_readout": _pre_update_readout,
    "erase_sign": _erase_sign,
    "transposed_state": _transposed_state,
    "no_decay_on_erase": _no_decay_on_erase,
}


# -------------------------------------------------------------------- pins

def pin_matches_per_channel_oracle(run):
    q, k, v, alpha, beta = _inputs(1, 23, 2, 5, 5)
    S0 = np.random.default_rng(2).standard_normal((3, 2, 5, 5))
    cu = [0, 9, 9, 23]
    o, ST = run(q, k, v, alpha, beta, S0, cu)
    ro, rST = kda_recurrent(q, k, v, np.repeat(alpha[:, :, None], 5, axis=2), beta, S0, cu_seqlens=cu)
    return _close(o, ro) and _close(ST, rST)


def pin_rotation_invariance(run):
    q, k, v, alpha, beta = _inputs(3, 17, 1, 4, 4)
    S0 = np.random.default_rng(4).standard_normal((1, 1, 4, 4))
    R, _ = np.linalg.qr(np.random.default_rng(5).standard_normal((4, 4)))
    o, ST = run(q, k, v, alpha, beta, S0)
    rot = lambda x: np.einsum("ij,thj->thi", R, x)
    o2, ST2 = run(rot(q), rot(k), v, alpha, beta, np.einsum("ij,nhjv->nhiv", R, S0))
    return _close(o2, o) and _close(ST2, np.einsum("ij,nhjv->nhiv", R, ST))


def pin_beta_zero_is_pure_decay(run):
    q, k, v, alpha, _ = _inputs(6, 12, 2, 3, 4)
    beta = np.zeros((12, 2))
    S0 = np.random.default_rng(7).standard_normal((1, 2, 3, 4))
    o, ST = run(q, k, v, alpha, beta, S0)
    g = np.cumprod(alpha, axis=0)                                     # [T, H]
    want_o = g[:, :, None] * np.einsum("hkv,thk->thv", S0[0], q)
    return _close(ST[0], g[-1][:, None, None] * S0[0]) and _close(o, want_o)


def pin_zero_rate_erases_history(run):
    q, k, v, alpha, beta = _inputs(8, 10, 2, 4, 3)
    alpha[6] = 0.0
    S0 = np.random.default_rng(9).standard_normal((1, 2, 4, 3))
    # tokens 0..6 only: after token 6 the state is beta_6 k_6 v_6^T
    o, ST = run(q[:7], k[:7], v[:7], alpha[:7], beta[:7], S0)
    want = beta[6][:, None, None] * _outer(k[6], v[6])
    return _close(ST[0], want) and _close(o[6], np.einsum("hkv,hk->hv", want, q[6]))


def pin_scalar_filter(run):
    T = 40
    rng = np.random.default_rng(10)
    a, b, kk = 0.8, 0.6, 0.9
    v = rng.standard_normal(T)
    ones = lambda x: np.full((T, 1), x)
    o, ST = run(ones(1.0)[:, :, None], ones(kk)[:, :, None], v[:, None, None], ones(a), ones(b))
    s = scipy.signal.lfilter([b * kk], [1.0, -a * (1.0 - b * kk * kk)], v)
    return _close(o[:, 0, 0], s) and _close(ST[0, 0, 0, 0], s[-1])


def pin_lms_step(run):
    q, k, v, _, beta = _inputs(11, 1, 1, 6, 3)
    S0 = np.random.default_rng(12).standard_normal((1, 1, 6, 3))
    o, ST = run(q, k, v, np.ones((1, 1)), beta, S0)
    S = S0[0, 0]
    grad = np.outer(k[0, 0], S.T @ k[0, 0] - v[0, 0])                 # d/dS 0.5 ||S^T k - v||^2
    return _close(ST[0, 0], S - beta[0, 0] * grad)


PINS = [pin_matches_per_channel_oracle, pin_rotation_invariance, pin_beta_zero_is_pure_decay,
        pin_zero_rate_erases_history, pin_scalar_filter, pin_lms_step]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    assert pin(oracle_runner)


def test_mutant_runner_matches_oracle_when_unbroken():
    def right(S, q, k, v, a, b):
        return gdn_step(S, q, k, v, a, b)
    assert all(pin(_mutant(right)) for pin in PINS)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    run = _mutant(MUTANTS[name])
    failed = []
    for pin in PINS:
        try:
            ok = pin(run)
        except Exception:  # a broken update may not even have the right shapes
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin catches {name}"


def test_per_channel_decay_breaks_rotation_invariance():
    """The rotation pin is specific to the scalar gate: KDA with different
    rates per key channel does not satisfy it."""
    q, k, v, _, beta = _inputs(13, 9, 1, 4, 4)
    alpha = np.random.default_rng(14).uniform(0.3, 1.0, (9, 1, 4))
    R, _ = np.linalg.qr(np.random.default_rng(15).standard_normal((4, 4)))
    o, _ = kda_recurrent(q, k, v, alpha, beta)
    rot = lambda x: np.einsum("ij,thj->thi", R, x)
    o2, _ = kda_recurrent(rot(q), rot(k), v, alpha, beta)
    assert np.max(np.abs(o2 - o)) > 1e-3


def test_decode_steps_equal_prefill():
    q, k, v, alpha, beta = _inputs(16, 6, 3, 8, 8)
    S0 = np.random.default_rng(17).standard_normal((1, 3, 8, 8))
    o, ST = gdn_recurrent(q, k, v, alpha, beta, S0)
    S = S0
    for t in range(6):
        ot, S = gdn_decode_step(q[t][None], k[t][None], v[t][None], alpha[t][None], beta[t][None], S)
        assert _close(ot[0], o[t])
    assert _close(S, ST)


def test_dense_batch_equals_varlen():
    q, k, v, alpha, beta = _inputs(18, 12, 2, 4, 4)
    a = gdn_recurrent(q, k, v, alpha, beta, num_seqs=3)
    b = gdn_recurrent(q, k, v, alpha, beta, cu_seqlens=[0, 4, 8, 12])
    assert _close(a[0], b[0]) and _close(a[1], b[1])


def test_rejects_per_channel_alpha():
    q, k, v, alpha, beta = _inputs(19, 4, 1, 4, 4)
    with pytest.raises(ValueError):
        gdn_recurrent(q, k, v, np.repeat(alpha[:, :, None], 4, axis=2), beta)
