"""The seeded input generators: deterministic, prefix-stable, right shapes and
distributions (CPU only)."""

import math

import torch

from gated_delta_rule_76_amd import inputs


def test_deterministic():
    a = inputs.token_inputs(100, 3, 16, torch.bfloat16, "strong", seed=5)
    b = inputs.token_inputs(100, 3, 16, torch.bfloat16, "strong", seed=5)
    for key in a:
        assert torch.equal(a[key], b[key])
    d = inputs.token_inputs(100, 3, 16, torch.bfloat16, "strong", seed=6)
    assert not torch.equal(d["q"], a["q"])


def test_distributions():
    x = inputs.token_inputs(4096, 4, 128, torch.float32, "strong", seed=0)
    norms = torch.linalg.vector_norm(x["k"], dim=-1)
    assert torch.allclose(norms, torch.ones_like(norms), atol=1e-5)
    assert x["alpha"].dtype == torch.float32 and x["beta"].dtype == torch.float32
    assert 0.10 < x["alpha"].mean().item() < 0.18          # exp(-softplus(N(0,1)+2))
    assert (x["alpha"] > 0).all() and (x["alpha"] < 1).all()
    assert abs(x["beta"].mean().item() - 0.5) < 0.01
    w = inputs.token_inputs(2048, 2, 64, torch.float32, "weak", seed=0)
    assert w["alpha"].mean().item() > 0.95
    m = inputs.token_inputs(2048, 2, 64, torch.float32, "medium", seed=0)
    assert 0.45 < m["alpha"].mean().item() < 0.55


def test_prefill_and_decode_packing():
    lens = inputs.varlen_lengths(8, 1024, 16384, seed=0)
    assert len(lens) == 8 and all(1024 <= L <= 16384 for L in lens)
    d = inputs.prefill_inputs([3, 0, 5], 2, 16, torch.float32, "medium", s0_std=0.02, seed=1)
    assert d["cu_seqlens"].tolist() == [0, 3, 3, 8]
    assert d["q"].shape == (8, 2, 16) and d["S0"].shape == (3, 2, 16, 16)
    assert abs(d["S0"].std().item() - 0.02) < 0.005
    dec = inputs.decode_inputs(4, 2, 16, steps=3, dtype=torch.bfloat16, seed=2)
    assert dec["q"].shape == (3, 4, 2, 16) and dec["beta"].shape == (3, 4, 2)
    assert dec["S"].shape == (4, 2, 16, 16)


def test_workloads_table():
    w = inputs.WORKLOADS
    assert w["prefill_4k"]["lengths"] == [4096] and w["prefill_4k"]["H"] == 32
    assert w["long_1m"]["lengths"] == [1 << 20]
    assert sum(inputs.workload_lengths(w["varlen_8seq"])) > 8 * 1024
    assert math.prod([w["decode_b256"]["B"], w["decode_b256"]["H"]]) == 8192


def test_scalar_gate_inputs():
    x = inputs.token_inputs(4096, 4, 64, torch.float32, "strong", seed=0, gate="head")
    assert x["alpha"].shape == (4096, 4)
    assert 0.10 < x["alpha"].mean().item() < 0.18
    c = inputs.token_inputs(4096, 4, 64, torch.float32, "strong", seed=0)
    assert torch.equal(x["q"], c["q"]) and torch.equal(x["v"], c["v"])   # only alpha differs
    d = inputs.decode_inputs(4, 2, 16, steps=3, seed=2, gate="head")
    assert d["alpha"].shape == (3, 4, 2)


def test_preact_inputs_are_what_the_final_inputs_are_made_from():
    f = inputs.token_inputs(512, 3, 32, torch.float32, "strong", seed=4)
    p = inputs.token_inputs(512, 3, 32, torch.float32, "strong", seed=4, form="preact")
    unit = lambda x: x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
    assert torch.allclose(unit(p["q"]), f["q"], atol=1e-6) and torch.allclose(unit(p["k"]), f["k"], atol=1e-6)
    assert torch.allclose(torch.exp(-torch.nn.functional.softplus(p["alpha"])), f["alpha"], rtol=1e-6)
    assert torch.allclose(torch.sigmoid(p["beta"]), f["beta"], rtol=1e-6)
    assert torch.equal(p["v"], f["v"])
