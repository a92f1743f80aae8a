"""The chunked backward model (tests/chunk_backward_model.py) against the
token-by-token backward oracle, on the CPU: the chunk-by-chunk reverse pass
and the per-chunk gradient products reproduce every gradient, across chunk
boundaries, ragged tails, varlen batches, both gate kinds and both decay
extremes."""

import numpy as np
import pytest

from oracle import rel_l2
from oracle.backward import kda_backward
from tests.chunk_backward_model import chunked_backward

NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dS0")


def _case(seed, lens, H, d, decay, per_head=False):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    q /= np.linalg.norm(q, axis=2, keepdims=True)
    k /= np.linalg.norm(k, axis=2, keepdims=True)
    v = rng.standard_normal((T, H, d))
    shift = {"strong": 2.0, "medium": 0.0, "weak": -4.0}[decay]
    ashape = (T, H) if per_head else (T, H, d)
    alpha = np.exp(-np.logaddexp(0.0, rng.standard_normal(ashape) + shift))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    N = len(lens)
    S0 = 0.3 * rng.standard_normal((N, H, d, d))
    dO = rng.standard_normal((T, H, d))
    dST = 0.1 * rng.standard_normal((N, H, d, d))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, alpha, beta, dO, S0, dST, cu


def _compare(args, tol=1e-10):
    q, k, v, alpha, beta, dO, S0, dST, cu = args
    want = kda_backward(q, k, v, alpha, beta, dO, S0, dST, cu_seqlens=cu)
    got = chunked_backward(q, k, v, alpha, beta, dO, S0, dST, cu_seqlens=cu)
    for name, g, w in zip(NAMES, got, want):
        e = rel_l2(g, w)
        assert e < tol, f"{name}: rel-L2 {e:.3e}"


@pytest.mark.parametrize("T", [1, 30, 64, 65, 150])
@pytest.mark.parametrize("decay", ["strong", "medium", "weak"])
def test_chunked_backward_matches_token_backward(T, decay):
    _compare(_case(T, [T], 1, 16, decay))


def test_chunked_backward_varlen_two_heads():
    _compare(_case(3, [40, 130, 1, 64], 2, 16, "medium"))


def test_chunked_backward_scalar_gate():
    _compare(_case(4, [70, 90], 2, 16, "medium", per_head=True))


def test_chunked_backward_wider_heads():
    _compare(_case(5, [129], 1, 32, "weak"))


def test_chunked_backward_exact_with_zero_rates():
    # rates of exactly 0 (history erased) at a chunk's first and last token,
    # mid-chunk, over a stretch of tokens, and tiny rates: the product form
    # never divides by a rate
    q, k, v, alpha, beta, dO, S0, dST, cu = _case(6, [150], 1, 16, "medium")
    alpha[0, 0, 3] = 0.0
    alpha[63, 0, 5] = 0.0
    alpha[64, 0, :] = 0.0
    alpha[90:95, 0, 7] = 0.0
    alpha[120, 0, 2] = 1e-30
    _compare((q, k, v, alpha, beta, dO, S0, dST, cu))


def test_chunked_backward_scalar_gate_zero_rate():
    q, k, v, alpha, beta, dO, S0, dST, cu = _case(7, [100], 2, 16, "strong", per_head=True)
    alpha[10, 0] = 0.0
    alpha[70, 1] = 0.0
    _compare((q, k, v, alpha, beta, dO, S0, dST, cu))
