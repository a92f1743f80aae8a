"""Decode step on the GPU (through the C ABI) against the fp64 oracle.

Tolerances: the decode kernel computes in fp32 from inputs that are exact in
fp32 (bf16 inputs widen exactly), so its results agree with the fp64 oracle
to fp32 rounding; 1e-5 rel-L2 is asserted for both input dtypes, well inside
the 2e-3 (bf16) / 1e-5 (fp32) targets.
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_76_amd import inputs, kda
from oracle import kda_decode_step, rel_l2
from tests.gpu_util import device, np64, seeded_sample

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_decode_matches_oracle_over_steps(D, dtype):
    dev = device()
    N, H, steps = 3, 2, 6
    d = inputs.decode_inputs(N, H, D, steps, dtype, "medium", s_std=0.5, seed=D, device=dev)
    S = d["S"].clone()
    S_ref = np64(S)
    for s in range(steps):
        o = kda.decode_step(d["q"][s], d["k"][s], d["v"][s], d["alpha"][s], d["beta"][s], S)
        ro, S_ref = kda_decode_step(np64(d["q"][s]), np64(d["k"][s]), np64(d["v"][s]),
                                    np64(d["alpha"][s]), np64(d["beta"][s]), S_ref)
        assert rel_l2(np64(o), ro) < 1e-5, (D, dtype, s)
    assert rel_l2(np64(S), S_ref) < 1e-5


def test_decode_identity_step_is_bit_exact():
    """alpha = 1, beta = 0 leaves the state bit-exact and reads o = S^T q."""
    dev = device()
    N, H, D = 4, 3, 128
    d = inputs.decode_inputs(N, H, D, 1, torch.bfloat16, "strong", seed=1, device=dev)
    S = d["S"].clone()
    ones = torch.ones_like(d["alpha"][0])
    zeros = torch.zeros_like(d["beta"][0])
    o = kda.decode_step(d["q"][0], d["k"][0], d["v"][0], ones, zeros, S)
    assert torch.equal(S, d["S"])
    ref = torch.einsum("nhk,nhkv->nhv", d["q"][0].double(), d["S"].double())
    assert rel_l2(np64(o), np64(ref)) < 1e-6


def test_decode_overwrite_reads_back_v():
    """alpha = 1, beta = 1, unit k, q = k: the step overwrites the value stored
    under k, so o = v."""
    dev = device()
    N, H, D = 2, 4, 64
    d = inputs.decode_inputs(N, H, D, 1, torch.float32, "strong", s_std=1.0, seed=2, device=dev)
    S = d["S"].clone()
    k = d["k"][0]
    o = kda.decode_step(k, k, d["v"][0], torch.ones_like(d["alpha"][0]),
                        torch.ones_like(d["beta"][0]), S)
    assert torch.allclose(o, d["v"][0], atol=2e-5)


def test_decode_workload_b256_100_steps():
    """The measured decode workload: B=256, H=32, d=128, bf16 q/k/v, state
    ~ 0.02 N(0,1), 100 consecutive in-place steps.  All outputs of a seeded
    sample of 256 (sequence, head) pairs are checked at every step, and their
    final states, against the oracle run on exactly those inputs."""
    dev = device()
    spec = inputs.WORKLOADS["decode_b256"]
    B, H, D, steps = spec["B"], spec["H"], spec["D"], spec["steps"]
    d = inputs.decode_inputs(B, H, D, steps, torch.bfloat16, "strong", s_std=0.02, seed=0, device=dev)
    pick = seeded_sample(B * H, 256, seed=3)
    bi, hi = pick // H, pick % H
    S = d["S"].clone()
    S_ref = np64(d["S"][bi, hi])
    o_all = torch.empty((steps, B, H, D), dtype=torch.float32, device=dev)
    for s in range(steps):
        kda.decode_step(d["q"][s], d["k"][s], d["v"][s], d["alpha"][s], d["beta"][s], S, out=o_all[s])
    got_o = np64(o_all[:, bi, hi])
    sel = {key: np64(d[key][:, bi, hi]) for key in ("q", "k", "v", "alpha", "beta")}
    worst = 0.0
    for s in range(steps):
        ro, S_ref = kda_decode_step(sel["q"][s], sel["k"][s], sel["v"][s], sel["alpha"][s],
                                    sel["beta"][s], S_ref)
        worst = max(worst, rel_l2(got_o[s], ro))
    assert worst < 2e-3 and worst < 1e-5, worst
    assert rel_l2(np64(S[bi, hi]), S_ref) < 1e-5


def test_decode_large_batch_streams_state():
    """B=1024 x 32 heads (2 GiB of state: the kernel reads it with
    non-temporal loads): three steps, every output and final state of a
    seeded sample of 128 (sequence, head) pairs against the oracle."""
    dev = device()
    B, H, D, steps = 1024, 32, 128, 3
    d = inputs.decode_inputs(B, H, D, steps, torch.bfloat16, "strong", 0.02, seed=3, device=dev)
    S = d["S"].clone()
    pick = seeded_sample(B * H, 128, seed=9)
    n_idx, h_idx = pick // H, pick % H
    S_ref = np64(d["S"][n_idx, h_idx])[:, None]
    for s in range(steps):
        o = kda.decode_step(d["q"][s], d["k"][s], d["v"][s], d["alpha"][s], d["beta"][s], S)
        sel = lambda t: np64(t[s][n_idx, h_idx])[:, None]
        ro, S_ref = kda_decode_step(sel(d["q"]), sel(d["k"]), sel(d["v"]), sel(d["alpha"]), sel(d["beta"]), S_ref)
        assert rel_l2(np64(o[n_idx, h_idx]), ro[:, 0]) < 1e-5, s
    assert rel_l2(np64(S[n_idx, h_idx]), S_ref[:, 0]) < 1e-5
