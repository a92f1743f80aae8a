"""Seeded random shapes through every GPU path against the fp64 oracle.

Each case draws the sequence count and lengths (around the 64-token chunk
edges and up to 300 tokens, empty sequences included), heads, head size,
q/k/v dtype, gate kind, input form, decay regime and initial state, then
checks prefill (o and S_T, rel-L2 over each whole tensor and over every
(sequence, head) slice), the backward pass (rel-L2 per gradient) or
multi-token verification (outputs, per-token states, live state untouched)
against the oracle on the same inputs, with the tolerances of the dedicated
tests: 2e-3 (bf16 prefill), 1e-5 (fp32 prefill, verification), 2e-5
(backward); the verification cases also check rollback by recomputation
(verify, accept, and both in one pass) against the history round bit for
bit.
"""

import random

import numpy as np
import pytest
import torch

from gated_delta_rule_76_amd import inputs, kda
from oracle import gdn_recurrent, kda_recurrent, rel_l2, speculative
from oracle.backward import kda_backward
from oracle.prologue import recurrent_from_preact
from tests.gpu_util import device, np64, parity

pytestmark = pytest.mark.gpu

CASES = 240


def _lengths(rng):
    pick = lambda: rng.choice([0, 1, 17, 63, 64, 65, 127, 128, 129, rng.randint(1, 300)])
    lens = [pick() for _ in range(rng.randint(1, 4))]
    if sum(lens) == 0:
        lens[0] = 5
    return lens


def _prefill_case(rng, dev, D, H, dtype, decay, seed):
    gate, form = rng.choice(["channel", "head"]), rng.choice(["final", "preact"])
    lens, s0 = _lengths(rng), rng.choice([None, 0.3])
    d = inputs.prefill_inputs(lens, H, D, dtype, decay, s0, seed=seed, device=dev, gate=gate, form=form)
    o, ST = kda.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"],
                        preact=form == "preact")
    S0 = None if d["S0"] is None else np64(d["S0"])
    args = (np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["alpha"]), np64(d["beta"]), S0)
    cu = np.asarray(d["cu_seqlens"].cpu())
    if form == "preact":
        ro, rS = recurrent_from_preact(*args, cu_seqlens=cu)
    else:
        ro, rS = (kda_recurrent if gate == "channel" else gdn_recurrent)(*args, cu_seqlens=cu)
    tol = 1e-5 if dtype == torch.float32 else 2e-3
    what = f"prefill lens={lens} {gate} {form} S0={s0}"
    try:
        rep = parity(o, ST, ro, rS, tol, what, cu)
    except AssertionError as e:
        return [(str(e), float("inf"), tol)]
    return [(what + " o, worst (seq, head)", rep["worst_o"][0], tol),
            (what + " S_T, worst (seq, head)", rep["worst_S_T"][0], tol)]


def _backward_case(rng, dev, D, H, dtype, decay, seed):
    gate, lens = rng.choice(["channel", "head"]), _lengths(rng)
    d = inputs.prefill_inputs(lens, H, D, dtype, decay, 0.3, seed=seed, device=dev, gate=gate)
    dO, dST = inputs.grad_inputs(sum(lens), H, D, len(lens), seed=seed, device=dev, dS_std=0.3)
    got = kda.backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dO, d["S0"], dST, d["cu_seqlens"])
    want = kda_backward(np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["alpha"]), np64(d["beta"]),
                        np64(dO), np64(d["S0"]), np64(dST), cu_seqlens=np.asarray(d["cu_seqlens"].cpu()))
    names = ("dq", "dk", "dv", "dalpha", "dbeta", "dS0")
    return [(f"backward lens={lens} {gate} {n}", rel_l2(np64(g), w), 2e-5) for n, g, w in zip(names, got, want)]


def _verify_case(rng, dev, D, H, dtype, decay, seed):
    B, K = rng.randint(1, 6), rng.randint(1, 6)
    x = inputs.decode_inputs(B * K, H, D, 1, dtype, decay, s_std=0.5, seed=seed, device=dev)
    tok = {n: x[n][0].reshape((B, K) + tuple(x[n].shape[2:])).contiguous()
           for n in ("q", "k", "v", "alpha", "beta")}
    S = x["S"][:B].clone()
    S0 = S.clone()
    o, hist = kda.decode_tokens(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S, keep_states=True)
    flat = lambda t: np64(t).reshape((-1,) + tuple(t.shape[2:]))
    ro, rst = speculative.decode_tokens(*(flat(tok[n]) for n in ("q", "k", "v", "alpha", "beta")), np64(S0), K)
    what = f"verify B={B} K={K}"
    # the rollback by recomputation against the history round, bit for bit
    # (accepted counts from the case's own seed, so the other cases keep their draws)
    acc = torch.from_numpy(np.random.RandomState(seed).randint(-1, K + 2, size=B).astype(np.int32)).to(dev)
    S_c = S0.clone()
    kda.state_commit(S_c, hist, acc)
    S_r = S0.clone()
    o_r = kda.verify_tokens(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S_r)
    same_verify = torch.equal(o_r, o) and torch.equal(S_r, S0)
    kda.accept_tokens(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], S_r, acc)
    # one pass: accept these tokens, then verify them again from the advanced state
    cur = tuple(tok[n] for n in ("q", "k", "v", "alpha", "beta"))
    S_f = S0.clone()
    o_f = kda.accept_verify_tokens(cur, acc, *cur, S_f)
    o_2 = kda.verify_tokens(*cur, S_r)
    return [(what + " o", rel_l2(np64(o).reshape(ro.shape), ro), 1e-5),
            (what + " states", rel_l2(np64(hist).reshape(rst.shape), rst), 1e-5),
            (what + " live state changed", float(not torch.equal(S, S0)), 0.5),
            (what + " verify_tokens differs from the history round", float(not same_verify), 0.5),
            (what + " accept_tokens differs from the commit", float(not torch.equal(S_r, S_c)), 0.5),
            (what + " accept_verify_tokens differs", float(not (torch.equal(S_f, S_r) and torch.equal(o_f, o_2))),
             0.5)]


def test_random_shapes_match_the_oracle():
    dev = device()
    rng = random.Random(2024)
    failures = []
    for i in range(CASES):
        kind = rng.choice([_prefill_case, _prefill_case, _backward_case, _verify_case])
        D, H = rng.choice([16, 32, 64, 128]), rng.randint(1, 5)
        dtype = rng.choice([torch.float32, torch.bfloat16])
        decay, seed = rng.choice(["strong", "medium", "weak"]), rng.randint(0, 10 ** 6)
        for what, err, tol in kind(rng, dev, D, H, dtype, decay, seed):
            if not err < tol:
                failures.append(f"case {i} D={D} H={H} {dtype} {decay} seed={seed}: {what} {err:.3e} (tol {tol})")
    assert not failures, "\n".join(failures[:20])
