"""Pre-activation inputs (KDA_INPUT_PREACT) on the GPU, through the C ABI,
against the fp64 oracle of the prologue followed by the recurrence
(oracle/prologue.py).

q and k arrive raw, alpha holds decay pre-activations a (alpha =
exp(-softplus(a))), beta holds b (beta = sigmoid(b)); the kernels form the
activated values in their load stage.  Tolerances as for the activated form:
rel-L2 1e-5 (fp32 q/k/v), 2e-3 (bf16), separately for o and S_T.  The oracle
consumes the exact tensors the GPU consumed.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_76_amd import inputs, kda
from oracle import rel_l2
from oracle.prologue import decode_step_from_preact, recurrent_from_preact
from tests.gpu_util import device, np64, parity, seeded_sample
from tests.oracle_pool import per_head

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-3}
GATES = {"channel": "channel", "head": "head"}


def _oracle(d, heads=None, cu=None, S0=None):
    sel = (lambda t: t) if heads is None else (lambda t: t[:, heads])
    return recurrent_from_preact(np64(sel(d["q"])), np64(sel(d["k"])), np64(sel(d["v"])),
                                 np64(sel(d["alpha"])), np64(sel(d["beta"])), S0, cu_seqlens=cu)


def _check(o, ST, ro, rST, tol, what, cu=None):
    parity(o, ST, ro, rST, tol, what, cu)


@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 65, 200])
def test_preact_prefill_sizes(gate, D, dtype, T):
    dev = device()
    d = inputs.prefill_inputs([T], 3, D, dtype, "medium", 0.5, seed=T + D, device=dev, gate=gate,
                              form="preact")
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], preact=True)
    ro, rST = _oracle(d, S0=np64(d["S0"]))
    _check(o, ST, ro, rST, TOL[dtype], f"{gate} D={D} T={T} {dtype}")


@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_preact_varlen_ragged_and_empty(gate, dtype):
    dev = device()
    lens = [0, 1, 63, 64, 65, 130, 0, 200]
    d = inputs.prefill_inputs(lens, 2, 64, dtype, "weak", 0.3, seed=31, device=dev, gate=gate,
                              form="preact")
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"],
                        preact=True)
    cu = np.asarray(d["cu_seqlens"].cpu())
    ro, rST = _oracle(d, cu=cu, S0=np64(d["S0"]))
    _check(o, ST, ro, rST, TOL[dtype], "varlen", cu)
    assert torch.equal(ST[0], d["S0"][0]) and torch.equal(ST[6], d["S0"][6])


@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_preact_extreme_values(gate, dtype):
    """Saturated pre-activations (alpha -> 0 or 1, beta -> 0 or 1, taking the
    direct path for blocks whose decay underflows), raw q and k of very
    different lengths, and all-zero q and k vectors (the 1e-12 floor keeps
    them zero)."""
    dev = device()
    d = inputs.prefill_inputs([150], 2, 64, dtype, "medium", 0.5, seed=32, device=dev, gate=gate,
                              form="preact")
    d["alpha"][5] = 90.0
    d["alpha"][70:74] = -90.0
    d["alpha"][100:102] = 30.0
    d["beta"][10:20] = 60.0
    d["beta"][20:30] = -60.0
    d["q"][40:60] *= 50.0
    d["k"][60:80] *= 0.01
    d["q"][90] = 0.0
    d["k"][91] = 0.0
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], preact=True)
    assert torch.isfinite(o).all() and torch.isfinite(ST).all()
    ro, rST = _oracle(d, S0=np64(d["S0"]))
    _check(o, ST, ro, rST, TOL[dtype], "extreme")


def test_preact_matches_activated_form():
    """The same layer fed the activated tensors (activated by torch in fp32)
    gives the same result to rounding."""
    dev = device()
    d = inputs.prefill_inputs([0, 77, 200], 4, 128, torch.float32, "strong", 0.1, seed=33,
                              device=dev, form="preact")
    o1, S1 = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"],
                         preact=True)
    unit = lambda x: torch.nn.functional.normalize(x, dim=-1, eps=1e-12)
    o2, S2 = kda.prefill(unit(d["q"]), unit(d["k"]), d["v"],
                         torch.exp(-torch.nn.functional.softplus(d["alpha"])).contiguous(),
                         torch.sigmoid(d["beta"]).contiguous(), d["S0"], d["cu_seqlens"])
    assert rel_l2(np64(o1), np64(o2)) < 1e-5 and rel_l2(np64(S1), np64(S2)) < 1e-5


@pytest.mark.parametrize("gate", ["channel", "head"])
def test_preact_prefill_4k_workload(gate):
    """B=1, H=32, T=4096, d=128, bf16 raw q/k, a = N(0,1) + 2, b = N(0,1):
    o of every token and head and every S_T."""
    dev = device()
    spec = inputs.WORKLOADS["prefill_4k"]
    d = inputs.prefill_inputs(spec["lengths"], spec["H"], spec["D"], torch.bfloat16, "strong", None,
                              seed=0, device=dev, gate=gate, form="preact")
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], preact=True)
    ro, rST = per_head(recurrent_from_preact, *(np64(d[x]) for x in ("q", "k", "v", "alpha", "beta")))
    _check(o, ST, ro, rST, 2e-3, f"preact prefill_4k {gate}")


@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_preact_decode_over_steps(gate, D, dtype):
    dev = device()
    N, H, steps = 3, 2, 6
    d = inputs.decode_inputs(N, H, D, steps, dtype, "medium", s_std=0.5, seed=D, device=dev, gate=gate,
                             form="preact")
    d["q"][2, 1, 0] = 0.0                                   # an all-zero raw q vector
    S = d["S"].clone()
    S_ref = np64(S)
    for s in range(steps):
        o = kda.decode_step(d["q"][s], d["k"][s], d["v"][s], d["alpha"][s], d["beta"][s], S,
                            preact=True)
        ro, S_ref = decode_step_from_preact(np64(d["q"][s]), np64(d["k"][s]), np64(d["v"][s]),
                                            np64(d["alpha"][s]), np64(d["beta"][s]), S_ref)
        assert rel_l2(np64(o), ro) < 1e-5, (gate, D, dtype, s)
    assert rel_l2(np64(S), S_ref) < 1e-5


def test_preact_decode_workload_b256():
    """B=256, H=32, d=128, bf16 raw q/k, 100 in-place steps: every output of
    a seeded sample of 256 (sequence, head) pairs, and their final states."""
    dev = device()
    B, H, D, steps = 256, 32, 128, 100
    d = inputs.decode_inputs(B, H, D, steps, torch.bfloat16, "strong", 0.02, seed=0, device=dev,
                             form="preact")
    S = d["S"].clone()
    pick = seeded_sample(B * H, 256, seed=6)
    n_idx, h_idx = pick // H, pick % H
    S_ref = np64(d["S"][n_idx, h_idx])[:, None]
    for s in range(steps):
        o = kda.decode_step(d["q"][s], d["k"][s], d["v"][s], d["alpha"][s], d["beta"][s], S,
                            preact=True)
        sel = lambda t: np64(t[s][n_idx, h_idx])[:, None]
        ro, S_ref = decode_step_from_preact(sel(d["q"]), sel(d["k"]), sel(d["v"]), sel(d["alpha"]),
                                            sel(d["beta"]), S_ref)
        assert rel_l2(np64(o[n_idx, h_idx]), ro[:, 0]) < 2e-3, s
    assert rel_l2(np64(S[n_idx, h_idx]), S_ref[:, 0]) < 2e-3


def test_preact_prefill_matches_decode_steps():
    dev = device()
    T, H, D = 70, 2, 128
    d = inputs.prefill_inputs([T], H, D, torch.bfloat16, "medium", 0.1, seed=34, device=dev,
                              form="preact")
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], preact=True)
    S = d["S0"].clone()
    outs = [kda.decode_step(d["q"][t:t + 1], d["k"][t:t + 1], d["v"][t:t + 1], d["alpha"][t:t + 1],
                            d["beta"][t:t + 1], S, preact=True) for t in range(T)]
    assert rel_l2(np64(torch.cat(outs)), np64(o)) < 2e-4
    assert rel_l2(np64(S), np64(ST)) < 2e-4
