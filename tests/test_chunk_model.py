"""The chunked algorithm (as a numpy model of the HIP prefill) against the
token-by-token oracle, on the CPU: exactness of the chunked rewrite, the tail
padding, the underflow fallback, and the error of split-bf16 operands."""

import numpy as np
import pytest
import torch

from oracle import kda_recurrent, rel_l2
from tests.chunk_model import chunked_prefill


def _case(seed, T, d, decay):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, d))
    shift = {"strong": 2.0, "medium": 0.0, "weak": -4.0}[decay]
    alpha = np.exp(-np.logaddexp(0.0, rng.standard_normal((T, d)) + shift))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    S0 = 0.5 * rng.standard_normal((d, d))
    return q, k, v, alpha, beta, S0


def _oracle(q, k, v, alpha, beta, S0):
    o, S = kda_recurrent(q[:, None], k[:, None], v[:, None], alpha[:, None], beta[:, None],
                         S0[None, None])
    return o[:, 0], S[0, 0]


@pytest.mark.parametrize("form", ["wy", "reassociated"])
@pytest.mark.parametrize("T", [1, 16, 63, 64, 65, 150])
@pytest.mark.parametrize("decay", ["strong", "medium", "weak"])
def test_chunked_rewrite_is_exact(T, decay, form):
    q, k, v, alpha, beta, S0 = _case(T, T, 16, decay)
    o, S = chunked_prefill(q, k, v, alpha, beta, S0, form=form)
    ro, rS = _oracle(q, k, v, alpha, beta, S0)
    assert rel_l2(o, ro) < 1e-12 and rel_l2(S, rS) < 1e-12


@pytest.mark.parametrize("form", ["wy", "reassociated"])
def test_zero_decay_takes_the_fallback_and_stays_exact(form):
    q, k, v, alpha, beta, S0 = _case(3, 130, 8, "medium")
    alpha[5, 2] = 0.0
    alpha[70:75, :] = 0.0
    alpha[100, 7] = 1e-35
    o, S = chunked_prefill(q, k, v, alpha, beta, S0, form=form)
    ro, rS = _oracle(q, k, v, alpha, beta, S0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert rel_l2(o, ro) < 1e-12 and rel_l2(S, rS) < 1e-12


def _split_bf16(x):
    """hi + lo bf16 representation (round to nearest even), as the kernels carry operands."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    hi = t.to(torch.bfloat16).to(torch.float32)
    lo = (t - hi).to(torch.bfloat16).to(torch.float32)
    return (hi + lo).double().numpy()


@pytest.mark.parametrize("form", ["wy", "reassociated"])
@pytest.mark.parametrize("decay", ["strong", "weak"])
def test_split_bf16_operands_meet_the_tolerance(decay, form):
    """Emulated operand rounding to a bf16 hi/lo pair keeps rel-L2 well below
    2e-3 at d = 128 (the drop of the lo*lo term is not modelled; it is below
    2^-16 relative)."""
    q, k, v, alpha, beta, S0 = _case(7, 200, 128, decay)
    bf = lambda x: torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    q, k, v = bf(q), bf(k), bf(v)
    o, S = chunked_prefill(q, k, v, alpha, beta, S0, round_operand=_split_bf16, form=form)
    ro, rS = _oracle(q, k, v, alpha, beta, S0)
    assert rel_l2(o, ro) < 2e-4 and rel_l2(S, rS) < 2e-4
