"""Pins for the multi-token / speculative-verification oracle,
oracle/speculative.py: its outputs and kept states must be the prefill
oracle's (independently written and pinned) over the same tokens, the
rollback must give the state after exactly the accepted tokens, and each
planted mistake below must fail a pin."""

import numpy as np
import pytest

from oracle import gdn_recurrent, kda_decode_step, kda_recurrent
from oracle import speculative as sp


def _case(seed, N, k, H, d, gate):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N * k, H, d))
    kk = rng.standard_normal((N * k, H, d))
    kk /= np.linalg.norm(kk, axis=-1, keepdims=True)
    v = rng.standard_normal((N * k, H, d))
    alpha = rng.uniform(0.3, 1.0, (N * k, H, d) if gate == "channel" else (N * k, H))
    beta = rng.uniform(0.0, 1.0, (N * k, H))
    S = rng.standard_normal((N, H, d, d))
    return q, kk, v, alpha, beta, S


def _prefix(case, N, k, j):
    """The prefill oracle over the first j tokens of every sequence."""
    q, kk, v, alpha, beta, S = case
    rows = np.concatenate([np.arange(n * k, n * k + j) for n in range(N)]).astype(int)
    run = kda_recurrent if alpha.ndim == 3 else gdn_recurrent
    return run(q[rows], kk[rows], v[rows], alpha[rows], beta[rows], S, num_seqs=N)


def pin_outputs_and_states_are_prefixes(dt, cm):
    N, k = 3, 4
    case = _case(1, N, k, 2, 5, "channel")
    o, states = dt(*case, k)
    full_o, _ = _prefix(case, N, k, k)
    ok = np.allclose(o, full_o, rtol=1e-12, atol=1e-12)
    for j in range(1, k + 1):
        _, ST = _prefix(case, N, k, j)
        ok = ok and np.allclose(states[:, j - 1], ST, rtol=1e-12, atol=1e-12)
    return ok


def pin_rollback_to_accepted(dt, cm):
    N, k = 4, 3
    case = _case(2, N, k, 2, 4, "head")
    _, states = dt(*case, k)
    accepted = np.array([0, 1, 3, 2])
    got = cm(case[5], states, accepted)
    ok = np.array_equal(got[0], case[5][0])
    for n in range(1, N):
        _, ST = _prefix(case, N, k, int(accepted[n]))
        ok = ok and np.allclose(got[n], ST[n], rtol=1e-12, atol=1e-12)
    capped = cm(case[5], states, np.array([9, 9, 9, 9]))
    return ok and np.array_equal(capped, states[:, -1])


def pin_one_token_is_a_decode_step(dt, cm):
    case = _case(3, 5, 1, 3, 6, "channel")
    o, states = dt(*case, 1)
    ro, rS = kda_decode_step(*case)
    return np.allclose(o, ro, rtol=1e-13, atol=1e-13) and np.allclose(states[:, 0], rS, rtol=1e-13,
                                                                      atol=1e-13)


PINS = [pin_outputs_and_states_are_prefixes, pin_rollback_to_accepted, pin_one_token_is_a_decode_step]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    assert pin(sp.decode_tokens, sp.commit)


def _commit_off_by_one(S, states, accepted):
    S = np.array(S, dtype=np.float64)
    for n, j in enumerate(accepted):
        j = min(int(j), states.shape[1] - 1)
        if j >= 1:
            S[n] = states[n, j]
    return S


def _states_before_update(q, k, v, alpha, beta, S, kk):
    o, states = sp.decode_tokens(q, k, v, alpha, beta, S, kk)
    shifted = np.concatenate([S[:, None], states[:, :-1]], axis=1)
    return o, shifted


def _tokens_interleaved(q, k, v, alpha, beta, S, kk):
    # reads token t of sequence n from row t*N + n instead of n*k + t
    N = S.shape[0]
    perm = np.array([t * N + n for n in range(N) for t in range(kk)])
    return sp.decode_tokens(q[perm], k[perm], v[perm], alpha[perm], beta[perm], S, kk)


MUTANTS = {
    "commit_off_by_one": (sp.decode_tokens, _commit_off_by_one),
    "states_before_update": (_states_before_update, sp.commit),
    "tokens_interleaved": (_tokens_interleaved, sp.commit),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    failed = [p.__name__ for p in PINS if not p(*MUTANTS[name])]
    assert failed, f"no pin catches {name}"


def test_input_state_is_not_modified():
    case = _case(4, 2, 3, 2, 4, "channel")
    S = case[5].copy()
    sp.decode_tokens(*case, 3)
    assert np.array_equal(S, case[5])
