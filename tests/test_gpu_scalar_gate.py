"""Scalar-gate (Gated DeltaNet) form on the GPU, through the C ABI, against
the fp64 scalar-gate oracle (oracle/scalar_gate.py).

alpha holds one rate per (token, head); the kernels are the KDA kernels with
the rate broadcast to every key channel, so besides the oracle they must
reproduce the per-channel path fed that broadcast: exactly for fp32 q/k/v and
for decode; for the bf16 prefill the scalar path keeps k and q exact in its
chunk records (Khat = Gamma k with one Gamma per token) where the
per-channel path carries Khat and Qhat as bf16 hi/lo pairs, so the two agree
to within that rounding (rel-L2 5e-5).  Tolerances against the oracle as for
KDA: rel-L2 1e-5 (fp32 q/k/v), 2e-3 (bf16), separately for o and S_T; the
oracle consumes the exact tensors the GPU consumed.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_76_amd import inputs, kda
from oracle import gdn_decode_step, gdn_recurrent, rel_l2
from tests.gpu_util import device, np64, parity, seeded_sample
from tests.oracle_pool import per_head

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-3}


def _oracle(d, heads=None, cu=None, S0=None):
    sel = (lambda t: t) if heads is None else (lambda t: t[:, heads])
    return gdn_recurrent(np64(sel(d["q"])), np64(sel(d["k"])), np64(sel(d["v"])),
                         np64(sel(d["alpha"])), np64(sel(d["beta"])), S0, cu_seqlens=cu)


def _check(o, ST, ro, rST, tol, what, cu=None):
    parity(o, ST, ro, rST, tol, what, cu)


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 65, 200])
def test_scalar_gate_prefill_sizes(D, dtype, T):
    dev = device()
    d = inputs.prefill_inputs([T], 3, D, dtype, "medium", 0.5, seed=T + D, device=dev, gate="head")
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    ro, rST = _oracle(d, S0=np64(d["S0"]))
    _check(o, ST, ro, rST, TOL[dtype], f"D={D} T={T} {dtype}")


@pytest.mark.parametrize("decay", ["strong", "weak"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_scalar_gate_decay_regimes(decay, dtype):
    dev = device()
    d = inputs.prefill_inputs([300], 4, 128, dtype, decay, 0.5, seed=21, device=dev, gate="head")
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    ro, rST = _oracle(d, S0=np64(d["S0"]))
    _check(o, ST, ro, rST, TOL[dtype], f"decay {decay}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_scalar_gate_equals_per_channel_broadcast(dtype):
    """The per-head rate broadcast to every key channel through the KDA path:
    the same bits for fp32 q/k/v and for decode; within the per-channel
    path's hi/lo rounding of Khat and Qhat for the bf16 prefill."""
    dev = device()
    d = inputs.prefill_inputs([0, 1, 65, 200], 3, 128, dtype, "medium", 0.3, seed=22,
                              device=dev, gate="head")
    wide = d["alpha"][:, :, None].expand(d["q"].shape).contiguous()
    args = (d["q"], d["k"], d["v"])
    o1, S1 = kda.prefill(*args, d["alpha"], d["beta"], d["S0"], d["cu_seqlens"])
    o2, S2 = kda.prefill(*args, wide, d["beta"], d["S0"], d["cu_seqlens"])
    if dtype == torch.float32:
        assert torch.equal(o1, o2) and torch.equal(S1, S2)
    else:
        assert rel_l2(np64(o1), np64(o2)) < 5e-5 and rel_l2(np64(S1), np64(S2)) < 5e-5
    for t in range(3):
        S_a, S_b = d["S0"].clone(), d["S0"].clone()
        x = lambda key: d[key][t:t + 4].contiguous()
        oa = kda.decode_step(x("q"), x("k"), x("v"), x("alpha"), x("beta"), S_a)
        ob = kda.decode_step(x("q"), x("k"), x("v"), wide[t:t + 4].contiguous(), x("beta"), S_b)
        assert torch.equal(oa, ob) and torch.equal(S_a, S_b)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_scalar_gate_varlen_ragged_and_empty(dtype):
    dev = device()
    lens = [0, 1, 63, 64, 65, 130, 0, 200]
    d = inputs.prefill_inputs(lens, 2, 64, dtype, "medium", 0.3, seed=23, device=dev, gate="head")
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"])
    cu = np.asarray(d["cu_seqlens"].cpu())
    ro, rST = _oracle(d, cu=cu, S0=np64(d["S0"]))
    _check(o, ST, ro, rST, TOL[dtype], "varlen", cu)
    assert torch.equal(ST[0], d["S0"][0]) and torch.equal(ST[6], d["S0"][6])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_scalar_gate_zero_rate(dtype):
    """alpha = 0 erases a head's history; a block whose decay falls below
    2^-100 takes the direct path for its diagonal tile."""
    dev = device()
    d = inputs.prefill_inputs([150], 2, 64, dtype, "medium", 0.5, seed=24, device=dev, gate="head")
    d["alpha"][5, 0] = 0.0
    d["alpha"][70:74, 1] = 0.0
    d["alpha"][100, :] = 1e-35
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    assert torch.isfinite(o).all() and torch.isfinite(ST).all()
    ro, rST = _oracle(d, S0=np64(d["S0"]))
    _check(o, ST, ro, rST, TOL[dtype], "zero rate")


def test_scalar_gate_prefill_4k_workload():
    """B=1, H=32, T=4096, d=128, bf16, alpha = exp(-softplus(N(0,1)+2)) per
    (token, head): o of every token and head and every S_T."""
    dev = device()
    spec = inputs.WORKLOADS["prefill_4k"]
    d = inputs.prefill_inputs(spec["lengths"], spec["H"], spec["D"], torch.bfloat16, "strong", None,
                              seed=0, device=dev, gate="head")
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    ro, rST = per_head(gdn_recurrent, *(np64(d[x]) for x in ("q", "k", "v", "alpha", "beta")))
    _check(o, ST, ro, rST, 2e-3, "scalar-gate prefill_4k")


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_scalar_gate_decode_over_steps(D, dtype):
    dev = device()
    N, H, steps = 3, 2, 6
    d = inputs.decode_inputs(N, H, D, steps, dtype, "medium", s_std=0.5, seed=D, device=dev, gate="head")
    S = d["S"].clone()
    S_ref = np64(S)
    for s in range(steps):
        o = kda.decode_step(d["q"][s], d["k"][s], d["v"][s], d["alpha"][s], d["beta"][s], S)
        ro, S_ref = gdn_decode_step(np64(d["q"][s]), np64(d["k"][s]), np64(d["v"][s]),
                                    np64(d["alpha"][s]), np64(d["beta"][s]), S_ref)
        assert rel_l2(np64(o), ro) < 1e-5, (D, dtype, s)
    assert rel_l2(np64(S), S_ref) < 1e-5


def test_scalar_gate_decode_workload_b256():
    """B=256, H=32, d=128, bf16, 100 in-place steps: every output of a seeded
    sample of 256 (sequence, head) pairs, and their final states."""
    dev = device()
    B, H, D, steps = 256, 32, 128, 100
    d = inputs.decode_inputs(B, H, D, steps, torch.bfloat16, "strong", 0.02, seed=0, device=dev,
                             gate="head")
    S = d["S"].clone()
    pick = seeded_sample(B * H, 256, seed=4)
    n_idx, h_idx = pick // H, pick % H
    S_ref = np64(d["S"][n_idx, h_idx])[:, None]
    for s in range(steps):
        o = kda.decode_step(d["q"][s], d["k"][s], d["v"][s], d["alpha"][s], d["beta"][s], S)
        sel = lambda t: np64(t[s][n_idx, h_idx])[:, None]
        ro, S_ref = gdn_decode_step(sel(d["q"]), sel(d["k"]), sel(d["v"]), sel(d["alpha"]),
                                    sel(d["beta"]), S_ref)
        assert rel_l2(np64(o[n_idx, h_idx]), ro[:, 0]) < 2e-3, s
    assert rel_l2(np64(S[n_idx, h_idx]), S_ref[:, 0]) < 2e-3


def test_scalar_gate_prefill_matches_decode_steps():
    dev = device()
    T, H, D = 70, 2, 128
    d = inputs.prefill_inputs([T], H, D, torch.bfloat16, "medium", 0.1, seed=25, device=dev, gate="head")
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    S = d["S0"].clone()
    outs = [kda.decode_step(d["q"][t:t + 1], d["k"][t:t + 1], d["v"][t:t + 1], d["alpha"][t:t + 1],
                            d["beta"][t:t + 1], S) for t in range(T)]
    assert rel_l2(np64(torch.cat(outs)), np64(o)) < 2e-4
    assert rel_l2(np64(S), np64(ST)) < 2e-4
