"""The kernels stay inside the rows they are given.

Ragged tails are handled by clamped row indices and by buffer descriptors
sized to a chunk's valid rows (loads past them return zero, stores past them
are dropped by the hardware).  These tests place every input and output of a
call at the front of a larger allocation whose remaining rows hold NaN: a
load past the valid rows would carry a NaN into the results, a store past
them would overwrite the guard.  Each call must give exactly (bit for bit)
what the same call gives on tight tensors, and leave every guard row as it
was.  (All accesses stay inside the allocations either way: the guards are
part of them.)
"""

import math

import pytest
import torch

from gated_delta_rule_76_amd import inputs, kda
from tests.gpu_util import device

pytestmark = pytest.mark.gpu

GUARD = 80  # rows past the end: more than one 64-token chunk


def _guarded(t, rows=GUARD):
    """t's values at the front of a tensor with `rows` more rows of NaN
    (float) or of a fixed bit pattern (int); returns (view, whole)."""
    whole = torch.empty((t.shape[0] + rows,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
    if t.dtype.is_floating_point:
        whole.fill_(math.nan)
    else:
        whole.fill_(0x5A5A5A5A)
    whole[: t.shape[0]].copy_(t)
    return whole[: t.shape[0]], whole


def _guard_intact(whole, n):
    g = whole[n:]
    if g.dtype.is_floating_point:
        return bool(torch.isnan(g).all())
    return bool((g == 0x5A5A5A5A).all())


@pytest.mark.parametrize("lengths", [[37], [64 * 3 + 5], [100, 29, 64, 1], [4096 + 37]])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_prefill_stays_inside_its_rows(lengths, dtype):
    dev = device()
    H, D = 3, 128 if dtype == torch.bfloat16 else 64
    d = inputs.prefill_inputs(lengths, H, D, dtype, "weak", 0.3, seed=len(lengths), device=dev)
    T = sum(lengths)
    cu = d["cu_seqlens"]
    o_ref, S_ref = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], cu)
    gq, gk, gv, ga, gb = (_guarded(d[n]) for n in ("q", "k", "v", "alpha", "beta"))
    o_view, o_whole = _guarded(torch.zeros_like(o_ref))
    o, S = kda.prefill(gq[0], gk[0], gv[0], ga[0], gb[0], d["S0"], cu, out=o_view)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    assert _guard_intact(o_whole, T)
    for view, whole in (gq, gk, gv, ga, gb):
        assert _guard_intact(whole, T)


def test_decode_step_stays_inside_its_rows():
    dev = device()
    N, H, D = 37, 3, 128
    x = inputs.decode_inputs(N, H, D, 1, torch.bfloat16, "strong", s_std=0.5, seed=5, device=dev)
    tok = {n: x[n][0] for n in ("q", "k", "v", "alpha", "beta")}
    S_ref = x["S"].clone()
    o_ref = kda.decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S_ref)
    g = {n: _guarded(t) for n, t in tok.items()}
    S_view, S_whole = _guarded(x["S"].clone(), rows=2)
    o_view, o_whole = _guarded(torch.zeros_like(o_ref))
    o = kda.decode_step(*(g[n][0] for n in ("q", "k", "v", "alpha", "beta")), S_view, out=o_view)
    assert torch.equal(o, o_ref) and torch.equal(S_view, S_ref)
    assert _guard_intact(o_whole, N) and _guard_intact(S_whole, N)


def test_verification_rounds_stay_inside_their_rows():
    dev = device()
    N, K, H, D = 5, 3, 2, 128
    x = inputs.decode_inputs(N * K, H, D, 1, torch.bfloat16, "medium", s_std=0.5, seed=6, device=dev)
    tok = {n: x[n][0].reshape((N, K) + tuple(x[n].shape[2:])).contiguous() for n in ("q", "k", "v", "alpha", "beta")}
    names = ("q", "k", "v", "alpha", "beta")
    acc = torch.tensor([0, 1, 3, 2, 7], dtype=torch.int32, device=dev)
    S0 = x["S"][:N].contiguous()
    # tight tensors
    S_ref = S0.clone()
    o_ref = kda.verify_tokens(*(tok[n] for n in names), S_ref)
    kda.accept_tokens(*(tok[n] for n in names), S_ref, acc)
    S_ref2 = S0.clone()
    o_ref2 = kda.accept_verify_tokens(tuple(tok[n] for n in names), acc, *(tok[n] for n in names), S_ref2)
    # guarded (GUARD extra sequences of NaN after each input, 2 after the states and outputs)
    g = {n: _guarded(tok[n]) for n in names}
    acc_view, acc_whole = _guarded(acc, rows=3)
    S_view, S_whole = _guarded(S0.clone(), rows=2)
    o_view, o_whole = _guarded(torch.zeros_like(o_ref), rows=2)
    o = kda.verify_tokens(*(g[n][0] for n in names), S_view, out=o_view)
    assert torch.equal(o, o_ref) and _guard_intact(o_whole, N)
    kda.accept_tokens(*(g[n][0] for n in names), S_view, acc_view)
    assert torch.equal(S_view, S_ref) and _guard_intact(S_whole, N)
    S_view.copy_(S0)
    o = kda.accept_verify_tokens(tuple(g[n][0] for n in names), acc_view, *(g[n][0] for n in names), S_view,
                                 out=o_view)
    assert torch.equal(o, o_ref2) and torch.equal(S_view, S_ref2)
    assert _guard_intact(o_whole, N) and _guard_intact(S_whole, N) and _guard_intact(acc_whole, N)


@pytest.mark.parametrize("lengths", [[37, 64 + 5], [300]])
def test_backward_stays_inside_its_rows(lengths):
    dev = device()
    H, D = 2, 128
    d = inputs.prefill_inputs(lengths, H, D, torch.bfloat16, "medium", 0.3, seed=7, device=dev)
    T = sum(lengths)
    dO, dST = inputs.grad_inputs(T, H, D, len(lengths), seed=7, device=dev, dS_std=0.3)
    cu = d["cu_seqlens"]
    ref = kda.backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dO, d["S0"], dST, cu)
    g = {n: _guarded(d[n]) for n in ("q", "k", "v", "alpha", "beta")}
    gO = _guarded(dO)
    got = kda.backward(*(g[n][0] for n in ("q", "k", "v", "alpha", "beta")), gO[0], d["S0"], dST, cu)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
