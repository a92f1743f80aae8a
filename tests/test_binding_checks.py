"""Host-side argument checks of the Python binding, without a GPU.

Outputs that the caller supplies (``out``, ``final_state``) must have exactly
the shape the call writes: a smaller buffer would be written past its end on
the device.  These tests replace the binding's device check with one that
accepts CPU tensors and make any library call fail, so they show that a wrong
shape is rejected on the host before anything reaches the C ABI.
"""

import pytest
import torch

from gated_delta_rule_76_amd import kda


@pytest.fixture
def host_only(monkeypatch):
    def require(name, t, dtype=None):
        if not isinstance(t, torch.Tensor):
            raise TypeError(name)
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} dtype")
        if not t.is_contiguous():
            raise ValueError(f"{name} contiguity")

    def no_library():
        raise AssertionError("the library was reached before the shape check")

    monkeypatch.setattr(kda, "_require_gpu", require)
    monkeypatch.setattr(kda, "lib", no_library)


def _prefill_inputs(T=70, H=2, D=16):
    g = torch.Generator().manual_seed(0)
    q, k, v = (torch.randn(T, H, D, generator=g) for _ in range(3))
    alpha = torch.rand(T, H, D, generator=g)
    beta = torch.rand(T, H, generator=g)
    return q, k, v, alpha, beta


def test_prefill_rejects_short_out(host_only):
    q, k, v, a, b = _prefill_inputs()
    with pytest.raises(ValueError, match="out has shape"):
        kda.prefill(q, k, v, a, b, out=torch.empty(69, 2, 16))


def test_prefill_rejects_wrong_final_state(host_only):
    q, k, v, a, b = _prefill_inputs()
    with pytest.raises(ValueError, match="final_state has shape"):
        kda.prefill(q, k, v, a, b, final_state=torch.empty(1, 2, 16, 8))


def test_decode_step_rejects_short_out(host_only):
    N, H, D = 4, 2, 16
    q, k, v = (torch.randn(N, H, D) for _ in range(3))
    S = torch.zeros(N, H, D, D)
    with pytest.raises(ValueError, match="out has shape"):
        kda.decode_step(q, k, v, torch.rand(N, H, D), torch.rand(N, H), S, out=torch.empty(N, H, D - 1))


def test_decode_tokens_rejects_short_out(host_only):
    N, K, H, D = 3, 2, 2, 16
    q, k, v = (torch.randn(N, K, H, D) for _ in range(3))
    S = torch.zeros(N, H, D, D)
    with pytest.raises(ValueError, match="out has shape"):
        kda.decode_tokens(q, k, v, torch.rand(N, K, H, D), torch.rand(N, K, H), S,
                          out=torch.empty(N, K, H, D // 2))


def test_decode_tokens_rejects_wrong_history(host_only):
    N, K, H, D = 3, 2, 2, 16
    q, k, v = (torch.randn(N, K, H, D) for _ in range(3))
    S = torch.zeros(N, H, D, D)
    with pytest.raises(ValueError, match="states must be"):
        kda.decode_tokens(q, k, v, torch.rand(N, K, H, D), torch.rand(N, K, H), S, keep_states=True,
                          states=torch.empty(N, K - 1, H, D, D))


def test_tensors_of_one_call_must_share_a_device(host_only):
    # (the meta device stands in for a second GPU: nothing is launched)
    q, k, v, a, b = _prefill_inputs()
    with pytest.raises(ValueError, match="beta is on meta"):
        kda.prefill(q, k, v, a, b.to("meta"))
    with pytest.raises(ValueError, match="out is on meta"):
        kda.prefill(q, k, v, a, b, out=torch.empty(70, 2, 16, device="meta"))
    N, H, D = 4, 2, 16
    q, k, v = (torch.randn(N, H, D) for _ in range(3))
    S = torch.zeros(N, H, D, D, device="meta")
    with pytest.raises(ValueError, match="state is on meta"):
        kda.decode_step(q, k, v, torch.rand(N, H, D), torch.rand(N, H), S)


def _round_inputs(N=3, K=2, H=2, D=16, seed=0):
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn(N, K, H, D, generator=g) for _ in range(3))
    return q, k, v, torch.rand(N, K, H, D, generator=g), torch.rand(N, K, H, generator=g)


def test_verify_tokens_rejects_short_out(host_only):
    q, k, v, a, b = _round_inputs()
    with pytest.raises(ValueError, match="out has shape"):
        kda.verify_tokens(q, k, v, a, b, torch.zeros(3, 2, 16, 16), out=torch.empty(3, 2, 2, 8))


def test_accept_tokens_rejects_wrong_counts(host_only):
    q, k, v, a, b = _round_inputs()
    S = torch.zeros(3, 2, 16, 16)
    with pytest.raises(ValueError, match="accepted has shape"):
        kda.accept_tokens(q, k, v, a, b, S, torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="state has shape"):
        kda.accept_tokens(q, k, v, a, b, torch.zeros(3, 2, 16, 8), torch.zeros(3, dtype=torch.int32))


def test_accept_verify_rejects_mismatched_rounds(host_only):
    prev = _round_inputs(seed=1)
    q, k, v, a, b = _round_inputs(seed=2)
    S = torch.zeros(3, 2, 16, 16)
    acc = torch.zeros(3, dtype=torch.int32)
    # the previous round with more tokens per sequence than this one
    longer = _round_inputs(K=3, seed=3)
    with pytest.raises(ValueError, match="previous round"):
        kda.accept_verify_tokens(longer, acc, q, k, v, a, b, S)
    with pytest.raises(ValueError, match="out has shape"):
        kda.accept_verify_tokens(prev, acc, q, k, v, a, b, S, out=torch.empty(3, 2, 2, 15))
    with pytest.raises(ValueError, match="accepted has shape"):
        kda.accept_verify_tokens(prev, torch.zeros(2, dtype=torch.int32), q, k, v, a, b, S)
