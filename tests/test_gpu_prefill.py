"""Chunked prefill on the GPU (through the C ABI) against the fp64 oracle.

Tolerances (rel-L2 over the whole tensor, separately for o and S_T):
  fp32 q/k/v  -> 1e-5 (fp32 matrix-core products, fp32 accumulation);
  bf16 q/k/v  -> 2e-3 (the layer's target; operands are carried as bf16
                 hi/lo pairs, about 16 significand bits, accumulation fp32).
The oracle always consumes the exact tensors the GPU consumed, copied back.
Sizes span several chunks and ragged tails; the measured workloads are
checked at full size on seeded samples of heads/windows (history older than
~1000 tokens has weight below 1e-300 under their decay, so a window run from
zero reproduces the state exactly).
"""

import numpy as np
import pytest
import torch

from gated_delta_rule_76_amd import inputs, kda
from oracle import kda_recurrent, rel_l2
from tests.gpu_util import device, np64, seeded_sample

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-3}


def _oracle(d, heads=None, cu=None, S0=None):
    sel = (lambda t: t) if heads is None else (lambda t: t[:, heads])
    return kda_recurrent(np64(sel(d["q"])), np64(sel(d["k"])), np64(sel(d["v"])),
                         np64(sel(d["alpha"])), np64(sel(d["beta"])),
                         None if S0 is None else S0, cu_seqlens=cu)


def _check(o, ST, ro, rST, tol, what):
    eo, es = rel_l2(np64(o), ro), rel_l2(np64(ST), rST)
    assert eo < tol and es < tol, f"{what}: o {eo:.3e}  S_T {es:.3e}  (tol {tol})"
    return eo, es


def test_tiny_fp32_workload():
    """B=1, H=2, T=64, d=16, fp32, alpha = exp(-softplus(N(0,1))), S0 = 0."""
    dev = device()
    d = inputs.prefill_inputs([64], 2, 16, torch.float32, "medium", None, seed=0, device=dev)
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    ro, rST = _oracle(d)
    _check(o, ST, ro, rST, 1e-5, "tiny fp32")


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 64, 65, 200])
def test_prefill_sizes(D, dtype, T):
    dev = device()
    d = inputs.prefill_inputs([T], 3, D, dtype, "strong", 0.5, seed=T + D, device=dev)
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    ro, rST = _oracle(d, S0=np64(d["S0"]))
    _check(o, ST, ro, rST, TOL[dtype], f"D={D} T={T} {dtype}")


@pytest.mark.parametrize("decay", ["medium", "weak"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_prefill_decay_regimes(decay, dtype):
    dev = device()
    d = inputs.prefill_inputs([300], 4, 128, dtype, decay, 0.5, seed=11, device=dev)
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    ro, rST = _oracle(d, S0=np64(d["S0"]))
    _check(o, ST, ro, rST, TOL[dtype], f"decay {decay}")


def test_prefill_fp32_many_chunks_weak_decay():
    """fp32 path at d=128 over many chunks with the longest memory: two
    packed sequences (16 chunks + a 40-token tail, 5 chunks + 13), S0."""
    dev = device()
    d = inputs.prefill_inputs([1064, 333], 2, 128, torch.float32, "weak", 0.5, seed=23, device=dev)
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"])
    ro, rST = _oracle(d, cu=np.asarray(d["cu_seqlens"].cpu()), S0=np64(d["S0"]))
    _check(o, ST, ro, rST, 1e-5, "fp32 many chunks")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_prefill_varlen_ragged_and_empty(dtype):
    dev = device()
    lens = [0, 1, 63, 64, 65, 130, 0, 200]
    d = inputs.prefill_inputs(lens, 2, 64, dtype, "medium", 0.3, seed=5, device=dev)
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"])
    ro, rST = _oracle(d, cu=np.asarray(d["cu_seqlens"].cpu()), S0=np64(d["S0"]))
    _check(o, ST, ro, rST, TOL[dtype], "varlen")
    assert torch.equal(ST[0], d["S0"][0]) and torch.equal(ST[6], d["S0"][6])   # empty sequences


@pytest.mark.parametrize("D", [32, 128])
def test_prefill_dense_batch_layout(D):
    dev = device()
    d = inputs.prefill_inputs([100] * 3, 2, D, torch.bfloat16, "strong", 0.1, seed=6, device=dev)
    shp = lambda t: t.reshape((3, 100) + tuple(t.shape[1:]))
    o, ST = kda.prefill(shp(d["q"]), shp(d["k"]), shp(d["v"]), shp(d["alpha"]), shp(d["beta"]), d["S0"])
    ro, rST = _oracle(d, cu=np.asarray(d["cu_seqlens"].cpu()), S0=np64(d["S0"]))
    _check(o.reshape(300, 2, D), ST, ro, rST, 2e-3, "dense batch")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_prefill_zero_decay_fallback(dtype):
    """alpha = 0 (history erased) and decays below 2^-100 inside a 16-token
    block take the direct path for that block's diagonal tile."""
    dev = device()
    d = inputs.prefill_inputs([150], 2, 64, dtype, "medium", 0.5, seed=7, device=dev)
    d["alpha"][5, 0, 3] = 0.0
    d["alpha"][70:74, 1, :] = 0.0
    d["alpha"][100, :, 7] = 1e-35
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    assert torch.isfinite(o).all() and torch.isfinite(ST).all()
    ro, rST = _oracle(d, S0=np64(d["S0"]))
    _check(o, ST, ro, rST, TOL[dtype], "zero decay")


def test_prefill_identity_leaves_state_exact():
    """alpha = 1, beta = 0: S_T == S0 bit-exact and o = S0^T q."""
    dev = device()
    d = inputs.prefill_inputs([130], 2, 128, torch.bfloat16, "strong", 0.5, seed=8, device=dev)
    ones = torch.ones_like(d["alpha"])
    o, ST = kda.prefill(d["q"], d["k"], d["v"], ones, torch.zeros_like(d["beta"]), d["S0"])
    assert torch.equal(ST, d["S0"])
    ref = torch.einsum("thk,hkv->thv", d["q"].double(), d["S0"][0].double())
    assert rel_l2(np64(o), np64(ref)) < 2e-5


def test_prefill_in_place_state():
    dev = device()
    d = inputs.prefill_inputs([90], 2, 64, torch.bfloat16, "strong", 0.5, seed=9, device=dev)
    ref_o, ref_S = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    S = d["S0"].clone()
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S, final_state=S)
    assert ST.data_ptr() == S.data_ptr()
    assert torch.equal(o, ref_o) and torch.equal(S, ref_S)


@pytest.mark.parametrize("split", [64, 97])
def test_prefill_split_carry_matches_unsplit(split):
    """Prefill of [0, s) then [s, T) from the returned state equals one call."""
    dev = device()
    d = inputs.prefill_inputs([300], 2, 128, torch.bfloat16, "weak", 0.1, seed=10, device=dev)
    full_o, full_S = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    sl = lambda t, a, b: t[a:b].contiguous()
    o1, S1 = kda.prefill(sl(d["q"], 0, split), sl(d["k"], 0, split), sl(d["v"], 0, split),
                         sl(d["alpha"], 0, split), sl(d["beta"], 0, split), d["S0"])
    o2, S2 = kda.prefill(sl(d["q"], split, 300), sl(d["k"], split, 300), sl(d["v"], split, 300),
                         sl(d["alpha"], split, 300), sl(d["beta"], split, 300), S1)
    assert rel_l2(np64(torch.cat([o1, o2])), np64(full_o)) < 2e-4
    assert rel_l2(np64(S2), np64(full_S)) < 2e-4


def test_prefill_matches_decode_steps():
    """A T-token prefill and T decode steps give the same outputs and state."""
    dev = device()
    T, H, D = 70, 2, 128
    d = inputs.prefill_inputs([T], H, D, torch.bfloat16, "strong", 0.1, seed=12, device=dev)
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    S = d["S0"].clone()
    outs = []
    for t in range(T):
        outs.append(kda.decode_step(d["q"][t:t + 1], d["k"][t:t + 1], d["v"][t:t + 1],
                                    d["alpha"][t:t + 1], d["beta"][t:t + 1], S))
    assert rel_l2(np64(torch.cat(outs)), np64(o)) < 2e-4
    assert rel_l2(np64(S), np64(ST)) < 2e-4


def test_prefill_4k_workload():
    """B=1, H=32, T=4096, d=128, bf16, strong decay, S0 = 0: o and S_T of a
    seeded sample of 6 heads against the oracle over all 4096 tokens."""
    dev = device()
    spec = inputs.WORKLOADS["prefill_4k"]
    d = inputs.prefill_inputs(spec["lengths"], spec["H"], spec["D"], torch.bfloat16, "strong", None,
                              seed=0, device=dev)
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    heads = seeded_sample(spec["H"], 6, seed=1)
    ro, rST = _oracle(d, heads=heads)
    _check(o[:, heads], ST[:, heads], ro, rST, 2e-3, "prefill_4k")


def test_prefill_varlen_8seq_workload():
    """8 sequences, lengths uniform in [1024, 16384], H=32, d=128, bf16,
    S0 ~ 0.02 N(0,1).  For a seeded sample of 4 heads: the first 1024 tokens
    of every sequence from its S0, and (o of the last 512 tokens, S_T) from a
    run of the last 1024 tokens from zero, against the oracle."""
    dev = device()
    spec = inputs.WORKLOADS["varlen_8seq"]
    lens = inputs.workload_lengths(spec, seed=0)
    d = inputs.prefill_inputs(lens, spec["H"], spec["D"], torch.bfloat16, "strong", spec["s0_std"],
                              seed=0, device=dev)
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"])
    heads = seeded_sample(spec["H"], 4, seed=2)
    cu = np.asarray(d["cu_seqlens"].cpu())
    W = 1024
    for n in range(len(lens)):
        s, e = int(cu[n]), int(cu[n + 1])
        win = {key: d[key][s:s + W] for key in ("q", "k", "v", "alpha", "beta")}
        ro, _ = _oracle(win, heads=heads, S0=np64(d["S0"][n:n + 1, heads]))
        assert rel_l2(np64(o[s:s + W, heads]), ro) < 2e-3, n
        win = {key: d[key][e - W:e] for key in ("q", "k", "v", "alpha", "beta")}
        ro, rST = _oracle(win, heads=heads)
        # The window's first tokens still see the dropped history; from its
        # second half on, that history weighs < 1e-300.
        _check(o[e - W // 2:e, heads], ST[n:n + 1, heads], ro[W // 2:], rST, 2e-3,
               f"varlen seq {n} tail")


def test_two_phase_calls_equal_prefill():
    """kda_prefill_chunk_local then kda_prefill_state_pass == kda_prefill."""
    dev = device()
    d = inputs.prefill_inputs([0, 100, 37], 2, 128, torch.bfloat16, "strong", 0.1, seed=13, device=dev)
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"])
    ref_o, ref_S = kda.prefill(*args)
    call = kda.PrefillCall(*args)
    call.chunk_local()
    o, S = call.state_pass()
    assert torch.equal(o, ref_o) and torch.equal(S, ref_S)


def test_prefill_long_1m_workload():
    """B=1, H=32, T=2^20, d=128, bf16, strong decay, S0 = 0 (a 1M-token
    context; ~130 GB of device memory with the workspace).  For a seeded
    sample of 2 heads: o of the first 65,536 tokens against the oracle, and
    (o of the last 512 tokens, S_T) from a run of the last 1024 tokens from
    zero.  On all heads: the run split in halves at a chunk boundary (the
    second half from the first half's S_T) is bit-identical to one call."""
    dev = device()
    spec = inputs.WORKLOADS["long_1m"]
    T, H, D = spec["lengths"][0], spec["H"], spec["D"]
    d = inputs.prefill_inputs([T], H, D, torch.bfloat16, "strong", None, seed=0, device=dev)
    ws = torch.empty(kda.prefill_workspace_size(1, T, H, D), dtype=torch.uint8, device=dev)
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], workspace=ws)
    heads = seeded_sample(H, 2, seed=3)
    P, W = 65536, 1024
    ro, _ = _oracle({key: d[key][:P] for key in ("q", "k", "v", "alpha", "beta")}, heads=heads)
    eo = rel_l2(np64(o[:P, heads]), ro)
    assert eo < 2e-3, f"long_1m prefix: o {eo:.3e}"
    ro, rST = _oracle({key: d[key][T - W:] for key in ("q", "k", "v", "alpha", "beta")}, heads=heads)
    _check(o[T - W // 2:, heads], ST[:, heads], ro[W // 2:], rST, 2e-3, "long_1m tail")
    half = T // 2
    o2 = torch.empty_like(o)
    S1 = torch.empty_like(ST)
    first = {key: d[key][:half] for key in ("q", "k", "v", "alpha", "beta")}
    second = {key: d[key][half:] for key in ("q", "k", "v", "alpha", "beta")}
    kda.prefill(first["q"], first["k"], first["v"], first["alpha"], first["beta"], workspace=ws,
                out=o2[:half], final_state=S1)
    _, S2 = kda.prefill(second["q"], second["k"], second["v"], second["alpha"], second["beta"], S1,
                        workspace=ws, out=o2[half:])
    assert torch.equal(o2, o) and torch.equal(S2, ST)
