"""Pins for the gate and normalisation prologue, oracle/prologue.py.

What fixes it other than itself: library routines (scipy.special.expit for
the logistic function, torch.nn.functional.normalize in float64 for the L2
normalisation with the same 1e-12 floor), the closed form
exp(-softplus(a)) = 1 / (1 + e^a), special values, and invariants (scale
invariance of the normalisation, rates inside (0, 1)).  Every planted
mistake below fails at least one pin.
"""

import numpy as np
import pytest
import scipy.special
import torch

from oracle import prologue
from oracle import gdn_recurrent, kda_recurrent


def _rng(seed):
    return np.random.default_rng(seed)


# Pins take the three prologue functions, so that broken variants go through
# the same checks.
def pin_decay_closed_form(decay, strength, norm):
    a = np.concatenate([_rng(1).normal(2.0, 3.0, 200), [-50.0, -5.0, 0.0, 5.0, 50.0]])
    return np.allclose(decay(a), scipy.special.expit(-a), rtol=1e-13, atol=0)


def pin_decay_special_values(decay, strength, norm):
    v = decay(np.array([0.0, 800.0, -800.0]))
    return np.isclose(v[0], 0.5, rtol=1e-15) and v[1] == 0.0 and v[2] == 1.0


def pin_strength_logistic(decay, strength, norm):
    b = np.concatenate([_rng(2).normal(0.0, 3.0, 200), [-40.0, 0.0, 40.0]])
    return (np.allclose(strength(b), scipy.special.expit(b), rtol=1e-13, atol=0)
            and np.isclose(strength(np.array([0.0]))[0], 0.5, rtol=1e-15))


def pin_normalise_matches_library(decay, strength, norm):
    x = _rng(3).standard_normal((7, 3, 16)) * _rng(4).uniform(0.01, 100.0, (7, 3, 1))
    x[2, 1] = 0.0                                                      # zero vector -> zero
    want = torch.nn.functional.normalize(torch.from_numpy(x), dim=-1, eps=1e-12).numpy()
    got = norm(x)
    return np.all(np.isfinite(got)) and np.allclose(got, want, rtol=1e-14, atol=1e-300)


def pin_normalise_scale_invariant(decay, strength, norm):
    x = _rng(5).standard_normal((5, 2, 8))
    n = np.linalg.norm(norm(x), axis=-1)
    return np.allclose(norm(3.7 * x), norm(x), rtol=1e-14) and np.allclose(n, 1.0, rtol=1e-14)


PINS = [pin_decay_closed_form, pin_decay_special_values, pin_strength_logistic,
        pin_normalise_matches_library, pin_normalise_scale_invariant]
RIGHT = (prologue.decay_from_preact, prologue.strength_from_preact, prologue.l2_normalise)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_prologue_pin(pin):
    assert pin(*RIGHT)


MUTANTS = {
    "decay_sign": (lambda a: np.exp(np.logaddexp(0.0, a)), RIGHT[1], RIGHT[2]),
    "decay_is_sigmoid": (lambda a: scipy.special.expit(a), RIGHT[1], RIGHT[2]),
    "strength_sign": (RIGHT[0], lambda b: scipy.special.expit(-b), RIGHT[2]),
    "norm_over_heads": (RIGHT[0], RIGHT[1],
                        lambda x: x / np.maximum(np.linalg.norm(x, axis=-2, keepdims=True), 1e-12)),
    "norm_unguarded": (RIGHT[0], RIGHT[1], lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)),
    "norm_squared": (RIGHT[0], RIGHT[1],
                     lambda x: x / np.maximum(np.sum(x * x, axis=-1, keepdims=True), 1e-12)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    with np.errstate(all="ignore"):
        failed = [p.__name__ for p in PINS if not p(*MUTANTS[name])]
    assert failed, f"no pin catches {name}"


def test_preact_recurrence_is_the_recurrence_on_activated_inputs():
    rng = _rng(6)
    T, H, d = 37, 2, 8
    q, k, v = (rng.standard_normal((T, H, d)) * 3.0 for _ in range(3))
    a, b = rng.normal(2.0, 1.0, (T, H, d)), rng.standard_normal((T, H))
    S0 = rng.standard_normal((2, H, d, d))
    cu = [0, 20, 37]
    o, ST = prologue.recurrent_from_preact(q, k, v, a, b, S0, cu_seqlens=cu)
    qn, kn, alpha, beta = prologue.activate(q, k, a, b)
    ro, rST = kda_recurrent(qn, kn, v, alpha, beta, S0, cu_seqlens=cu)
    assert np.allclose(o, ro, rtol=0, atol=0) and np.allclose(ST, rST, rtol=0, atol=0)
    # one pre-activation per head selects the scalar gate
    ah = a[:, :, 0]
    o2, ST2 = prologue.recurrent_from_preact(q, k, v, ah, b, S0, cu_seqlens=cu)
    go, gST = gdn_recurrent(qn, kn, v, prologue.decay_from_preact(ah), beta, S0, cu_seqlens=cu)
    assert np.array_equal(o2, go) and np.array_equal(ST2, gST)


def test_preact_decode_matches_preact_prefill():
    rng = _rng(7)
    T, H, d = 5, 3, 4
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    a, b = rng.normal(0.0, 1.0, (T, H)), rng.standard_normal((T, H))
    S0 = rng.standard_normal((1, H, d, d))
    o, ST = prologue.recurrent_from_preact(q, k, v, a, b, S0)
    S = S0
    for t in range(T):
        ot, S = prologue.decode_step_from_preact(q[t][None], k[t][None], v[t][None], a[t][None],
                                                 b[t][None], S)
        assert np.allclose(ot[0], o[t], rtol=1e-12, atol=1e-12)
    assert np.allclose(S, ST, rtol=1e-12, atol=1e-12)
