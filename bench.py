"""Benchmark of the KDA layer on one MI355X: prefill tokens/s/layer and decode steps/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-decode]

A step is one kda_prefill call (varlen schedule, chunk-local kernel, state
pass) over one batch of the prefill workload; by default prefill_4k: B=1,
H=32, T=4096, d=128, bf16 q/k/v, fp32 alpha/beta/state/o, seeded synthetic
inputs resident in HBM.  Five input sets (each with its own outputs and
workspace) are rotated so that consecutive steps do not find their working
set in the 256 MB Infinity Cache.  W untimed steps, then K steps between
two synchronisations timed with HIP events on the launch stream.

Prints one JSON line: the prefill rate as ``value``; per-call median and
p10/p90; the roofline of the dominant kernel (the layer's algorithmic bytes,
1,796 per token and head, times the token-heads of one call, over that
kernel's event-timed duration; ``traffic`` from the committed hardware
counter summary when it was taken on the current kernel source); the
matrix-core rate of the call (issued, from the committed counter summary of
the same source, and useful); the decode
rate (B=256, H=32, d=128, 100 in-place steps) with its own roofline; and the
fp64 CPU oracle timed on the host over the whole prefill_4k workload.

The line also carries, on the same prefill and decode shapes, the
scalar-gate form (one alpha per token and head) under ``scalar_gate`` and the
layer fed pre-activations (gate and normalisation computed in the kernels)
under ``preact``, speculative verification of two tokens per sequence
(kda_decode_tokens with the state history, then kda_state_commit) under
``verify``, and the backward pass over the prefill_4k workload under
``backward`` (``--no-variants`` skips all four).  ``--oracle-rates`` times only the CPU oracle, on every workload,
and prints those rates as one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
N_SETS = 5                     # input sets rotated between timed calls
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_prefill_4k.json")
KERNEL_SOURCE = os.path.join(ROOT, "gated_delta_rule_76_amd", "csrc", "kda_prefill.hip")
DECODE_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_decode_b%d.json")  # % batch
DECODE_SOURCE = os.path.join(ROOT, "gated_delta_rule_76_amd", "csrc", "kda_decode.hip")
MFMA_SUMMARY = os.path.join(ROOT, "profiles", "mfma_prefill_4k.json")
# the counter summaries of the prefill's variants on the same workload: the
# scalar gate and the pre-activation inputs (workload name + suffix)
VARIANT_SUFFIX = {("channel", "final"): "", ("head", "final"): "_head", ("channel", "preact"): "_preact"}


def _variant_path(path, suffix):
    return path[:-len(".json")] + suffix + ".json" if suffix else path
BACKWARD_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_backward_4k.json")
BACKWARD_SOURCE = os.path.join(ROOT, "gated_delta_rule_76_amd", "csrc", "kda_backward.hip")
VERIFY_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_verify_b%d_k%d.json")  # % (batch, tokens)
VERIFY_RECOMPUTE_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_verify_recompute_b%d_k%d.json")
VERIFY_FUSED_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_verify_fused_b%d_k%d.json")
DECODE_TOKENS_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_decode_tokens_b%d_k%d.json")
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores, TFLOP/s
# Useful matrix work of the chunked form per token and head at d = 128, C = 64:
# the decayed Gram blocks, the triangular transform and the state products
# counted once (no precision split), 139,264 flop.
USEFUL_FLOP_PER_TOKEN_HEAD = 139264
COPY_BYTES = 256 << 20         # --calibrate-copy: bytes read (and written) by the copy

WORKLOAD_TEXT = {
    "prefill_4k": "B=1 H=32 T=4096 d=128",
    "varlen_8seq": "8 seqs, lengths U[1024,16384], H=32 d=128, S0~0.02N",
    "long_1m": "B=1 H=32 T=1048576 d=128",
}


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="prefill_4k", choices=sorted(WORKLOAD_TEXT))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-variants", action="store_true",
                   help="skip the scalar-gate, pre-activation, verify and backward measurements")
    p.add_argument("--decode-batch", type=int, default=256)
    p.add_argument("--decode-large-batch", type=int, default=1024,
                   help="with the variants, also time the decode at this batch (2 GiB of state at "
                        "1024, eight times the Infinity Cache; 0 skips it)")
    p.add_argument("--bounded-workspace-mib", type=int, default=0,
                   help="also time the prefill with a workspace of this many MiB (in stripes when "
                        "less than the recommended size)")
    p.add_argument("--bounded-backward-mib", type=int, default=0,
                   help="also time the backward with a workspace of this many MiB (in pieces when "
                        "less than the recommended size)")
    p.add_argument("--oracle-rates", action="store_true",
                   help="only time the fp64 CPU oracle on every workload (no GPU)")
    p.add_argument("--only", choices=["backward", "verify", "verify_recompute", "verify_fused", "prefill_head",
                                      "prefill_preact", "decode_tokens"],
                   help="run only this leg (after --calibrate-copy, if given) and print its summary; "
                        "for hardware counter runs of one kernel family")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run a plain elementwise float64 copy of 256 MiB (a kernel of "
                        "known size for scaling hardware byte counters)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# Algorithmic bytes per token and head (d = 128, bf16 q/k/v, fp32 rest).
#   layer:        q, k, v (768) + alpha (512) + beta (4) + o (512)
#   chunk-local:  q, k (512) + alpha (512) + beta (4) read; record written
#   state pass:   record read; v (256) read; o (512) written
# The record is the chunk-local kernel's output per 64 tokens and head,
# read once by the state pass (its d/16 workgroups per head share it in L2).
# ---------------------------------------------------------------------------
# Decode: state read + write, q, k, v, alpha, beta, o per (sequence, head) and step.
# Scalar gate (one alpha per token and head): alpha is 4 bytes instead of 512.
ALPHA_BYTES = {"channel": 512, "head": 4}


def layer_bytes(gate):
    return 768 + ALPHA_BYTES[gate] + 4 + 512


def decode_bytes(gate):
    return 2 * 128 * 128 * 4 + 768 + ALPHA_BYTES[gate] + 4 + 512


def backward_bytes():
    """Per token and head: q, k, v (bf16), alpha, beta, dO read; dq, dk, dv,
    dalpha, dbeta written (fp32)."""
    return 768 + 512 + 4 + 512 + 4 * 512 + 4


def verify_bytes(k):
    """k tokens of one (sequence, head) with the state history: the state
    read once, k states written, each token's q, k, v, alpha, beta, o."""
    return 128 * 128 * 4 * (1 + k) + k * (768 + 512 + 4 + 512)


def record_bytes_per_token(d):
    from gated_delta_rule_76_amd import kda
    # one sequence of 64 tokens, one head: schedule table (256 B) + 2 records
    rec = (kda.prefill_workspace_size(1, 64, 1, d) - 256) // 2
    return rec / 64.0


def exact_record_bytes_per_token(d):
    """Record of the scalar-gate form with bf16 q/k: k and q as single bf16
    fragments (1 KiB each: 4 row tiles x d/32 k-blocks), Ktil^T T (d/16 x 2
    fragments of 2 KiB), the six M T fragments, Gamma_C (d floats) and the two
    per-token factors (2 x 64 floats), 256-byte aligned."""
    nkb = max(d, 32) // 32
    raw = 2 * 4 * nkb * 1024 + (d // 16) * 2 * 2048 + 6 * 2048 + 4 * d + 2 * 64 * 4
    return (-(-raw // 256) * 256) / 64.0


def kernel_bytes(d, gate="channel"):
    # (the scalar-gate form keeps exact k and q in its records: bf16 inputs)
    rb = exact_record_bytes_per_token(d) if gate == "head" else record_bytes_per_token(d)
    return {"chunk_local_kernel": 512 + ALPHA_BYTES[gate] + 4 + rb, "chunk_state_kernel": rb + 256 + 512}


def _events():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def bench_bounded(name, steps, warmup, dev, ws_bytes):
    """The prefill of workload ``name`` with a workspace of ws_bytes (the
    same inputs as bench_prefill's first set): ms per call over ``steps``
    back-to-back calls, and the stripes that workspace takes."""
    from gated_delta_rule_76_amd import inputs, kda
    spec = inputs.WORKLOADS[name]
    lens = inputs.workload_lengths(spec, seed=0)
    H, D = spec["H"], spec["D"]
    d = inputs.prefill_inputs(lens, H, D, torch.bfloat16, spec["decay"], spec["s0_std"], seed=0, device=dev)
    cu = d["cu_seqlens"] if len(lens) > 1 else None
    call = kda.PrefillCall(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], cu,
                           workspace_bytes=ws_bytes)
    for _ in range(warmup):
        call.run()
    e0, e1 = _events()
    e0.record()
    for _ in range(steps):
        call.run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    N, total = len(lens), sum(lens)
    table = -(-4 * (N + 1) // 256) * 256
    chunk_bytes = H * kda.record_bytes(D)
    W = (ws_bytes - table) // chunk_bytes          # S_T is written, so no carry area
    need = total // 64 + N if cu is not None else N * -(-lens[0] // 64)
    return {"workspace_bytes": ws_bytes, "chunks_per_stripe": int(min(W, need)),
            "stripes": int(-(-need // min(W, need))), "ms": ms,
            "value": total / (ms * 1e-3), "unit": "tokens/s/layer"}


def bench_prefill(name, steps, warmup, dev, gate="channel", form="final"):
    from gated_delta_rule_76_amd import inputs, kda
    spec = inputs.WORKLOADS[name]
    lens = inputs.workload_lengths(spec, seed=0)
    H, D = spec["H"], spec["D"]
    n_sets = N_SETS if sum(lens) <= 65536 else 1
    calls = []
    for s in range(n_sets):
        d = inputs.prefill_inputs(lens, H, D, torch.bfloat16, spec["decay"], spec["s0_std"],
                                  seed=s, device=dev, gate=gate, form=form)
        cu = d["cu_seqlens"] if len(lens) > 1 else None
        calls.append(kda.PrefillCall(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], cu,
                                     preact=form == "preact"))
    total = sum(lens)
    for i in range(warmup):
        calls[i % n_sets].run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = _events()
    e0.record()
    for i in range(steps):
        calls[i % n_sets].run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    # Per-call and per-phase timing (events on the launch stream, which is
    # the current stream), in a second pass of the same K calls.
    evs = []
    for i in range(steps):
        a, b = _events()
        c = torch.cuda.Event(enable_timing=True)
        call = calls[i % n_sets]
        a.record()
        call.chunk_local()
        b.record()
        call.state_pass()
        c.record()
        evs.append((a, b, c))
    torch.cuda.synchronize()
    cl = np.array([a.elapsed_time(b) for a, b, _ in evs])
    sp = np.array([b.elapsed_time(c) for _, b, c in evs])
    per_call = cl + sp
    # Each phase's average over the calls, leaving out calls that took more
    # than three times the median (a stall of the device or the host between
    # the events, not kernel time; their count is reported).
    keep = per_call <= 3.0 * np.median(per_call)
    return {"total_tokens": total, "H": H, "D": D, "ms": ms, "wall_s": wall, "lengths": lens,
            "phases_ms": {"chunk_local": float(cl[keep].mean()), "state_pass": float(sp[keep].mean())},
            "stalled_calls": int((~keep).sum()),
            "call_ms": {"median": float(np.median(per_call)), "p10": float(np.percentile(per_call, 10)),
                        "p90": float(np.percentile(per_call, 90))}}


def bench_decode(B, dev, gate="channel", form="final"):
    from gated_delta_rule_76_amd import inputs, kda
    spec = inputs.WORKLOADS["decode_b256"]
    H, D = spec["H"], spec["D"]
    n = spec["steps"]
    d = inputs.decode_inputs(B, H, D, n, torch.bfloat16, spec["decay"], spec["s_std"],
                             seed=0, device=dev, gate=gate, form=form)
    pre = form == "preact"
    S = d["S"].clone()
    o = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    for s in range(10):
        kda.decode_step(d["q"][s % n], d["k"][s % n], d["v"][s % n], d["alpha"][s % n],
                        d["beta"][s % n], S, out=o, preact=pre)
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record()
    for s in range(n):
        kda.decode_step(d["q"][s], d["k"][s], d["v"][s], d["alpha"][s], d["beta"][s], S, out=o,
                        preact=pre)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    # Context for the decode roofline: torch's in-place elementwise scaling of
    # the same fp32 state (one read and one write of every byte, nothing else).
    for _ in range(3):
        S.mul_(0.5)
    e0.record()
    for _ in range(20):
        S.mul_(0.5)
    e1.record()
    torch.cuda.synchronize()
    rmw_gbs = 2 * S.numel() * 4 / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e9
    return {"B": B, "H": H, "D": D, "steps": n, "ms_per_step": ms, "state_rmw_gbs": rmw_gbs}


def bench_decode_context(B, dev, steps=1000):
    """The per-token cost does not grow with the tokens already seen: one
    state advanced by 10 + ``steps`` consecutive decode steps (cycling
    through the workload's 100 input sets), the first and the last 100 of the
    ``steps`` each timed by one event pair."""
    from gated_delta_rule_76_amd import inputs, kda
    spec = inputs.WORKLOADS["decode_b256"]
    H, D, n = spec["H"], spec["D"], spec["steps"]
    d = inputs.decode_inputs(B, H, D, n, torch.bfloat16, spec["decay"], spec["s_std"], seed=0, device=dev)
    S = d["S"].clone()
    o = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    step = lambda s: kda.decode_step(d["q"][s % n], d["k"][s % n], d["v"][s % n], d["alpha"][s % n],
                                     d["beta"][s % n], S, out=o)
    e = [_events() for _ in range(2)]
    warm = 10  # (untimed: the state's first reads are not cached yet)
    for s in range(warm + steps):
        if s == warm:
            e[0][0].record()
        if s == warm + 100:
            e[0][1].record()
        if s == warm + steps - 100:
            e[1][0].record()
        step(s)
    e[1][1].record()
    torch.cuda.synchronize()
    first, last = (a.elapsed_time(b) / 100 for a, b in e)
    return {"B": B, "steps": steps, "first_100_ms_per_step": first, "last_100_ms_per_step": last,
            "last_over_first": last / first}


def bench_verify(B, K, dev, steps=50):
    """Speculative verification of K tokens per sequence (the next token and
    K - 1 drafts): kda_decode_tokens with the state history, then
    kda_state_commit of a seeded accepted count per sequence.  Each figure is
    one event pair around ``steps`` back-to-back calls on the launch stream:
    verify + commit pairs (the step rate), then verify alone, then commit
    alone (the per-kernel times)."""
    from gated_delta_rule_76_amd import inputs, kda
    spec = inputs.WORKLOADS["decode_b256"]
    H, D = spec["H"], spec["D"]
    sets = []
    for i in range(N_SETS):
        d = inputs.decode_inputs(B * K, H, D, 1, torch.bfloat16, spec["decay"], spec["s_std"], seed=i,
                                 device=dev)
        sets.append({key: d[key][0].reshape((B, K) + tuple(d[key].shape[2:])).contiguous()
                     for key in ("q", "k", "v", "alpha", "beta")})
    S = inputs.state(B, H, D, spec["s_std"], seed=0, device=dev)
    o = torch.empty((B, K, H, D), dtype=torch.float32, device=dev)
    hist = torch.empty((B, K, H, D, D), dtype=torch.float32, device=dev)
    g = torch.Generator(device="cpu")
    g.manual_seed(0)
    accepted = torch.randint(0, K + 1, (B,), generator=g, dtype=torch.int32).to(dev)
    run = lambda t: kda.decode_tokens(t["q"], t["k"], t["v"], t["alpha"], t["beta"], S, keep_states=True,
                                      out=o, states=hist)
    commit = lambda: kda.state_commit(S, hist, accepted)
    for i in range(5):
        run(sets[i % N_SETS])
        commit()
    torch.cuda.synchronize()

    def timed(body):
        e0, e1 = _events()
        e0.record()
        for i in range(steps):
            body(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    pair = timed(lambda i: (run(sets[i % N_SETS]), commit()))
    vt = timed(lambda i: run(sets[i % N_SETS]))
    ct = timed(lambda i: commit())
    n_acc = int((accepted > 0).sum())
    return {"B": B, "K": K, "H": H, "step_ms": pair, "verify_ms": vt, "commit_ms": ct,
            "committed_seqs": n_acc}


def bench_verify_recompute(B, K, dev, steps=50):
    """Speculative verification with rollback by recomputation: kda_verify_tokens
    (outputs only, no state written), then kda_accept_tokens of the same
    seeded accepted counts as bench_verify.  One event pair around ``steps``
    back-to-back rounds, then around the verifies alone and the accepts alone."""
    from gated_delta_rule_76_amd import inputs, kda
    spec = inputs.WORKLOADS["decode_b256"]
    H, D = spec["H"], spec["D"]
    sets = []
    for i in range(N_SETS):
        d = inputs.decode_inputs(B * K, H, D, 1, torch.bfloat16, spec["decay"], spec["s_std"], seed=i,
                                 device=dev)
        sets.append({key: d[key][0].reshape((B, K) + tuple(d[key].shape[2:])).contiguous()
                     for key in ("q", "k", "v", "alpha", "beta")})
    S = inputs.state(B, H, D, spec["s_std"], seed=0, device=dev)
    o = torch.empty((B, K, H, D), dtype=torch.float32, device=dev)
    g = torch.Generator(device="cpu")
    g.manual_seed(0)
    accepted = torch.randint(0, K + 1, (B,), generator=g, dtype=torch.int32).to(dev)
    ver = lambda t: kda.verify_tokens(t["q"], t["k"], t["v"], t["alpha"], t["beta"], S, out=o)
    acc = lambda t: kda.accept_tokens(t["q"], t["k"], t["v"], t["alpha"], t["beta"], S, accepted)
    for i in range(5):
        ver(sets[i % N_SETS])
        acc(sets[i % N_SETS])
    torch.cuda.synchronize()

    def timed(body):
        e0, e1 = _events()
        e0.record()
        for i in range(steps):
            body(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    pair = timed(lambda i: (ver(sets[i % N_SETS]), acc(sets[i % N_SETS])))
    vt = timed(lambda i: ver(sets[i % N_SETS]))
    at = timed(lambda i: acc(sets[i % N_SETS]))
    n_acc = int((accepted > 0).sum())
    state = D * D * 4
    tok = K * (768 + 512 + 4 + 512)
    # bytes: verify reads each state once plus the tokens' inputs and outputs;
    # an accepting sequence's state is read and written once more, with the
    # inputs of its tokens (all k counted)
    v_bytes = B * H * (state + tok)
    a_bytes = n_acc * H * (2 * state + K * (768 + 512 + 4))
    gbs = (v_bytes + a_bytes) / (pair * 1e-3) / 1e9
    return {"metric": "speculative verify steps/s, rollback by recomputation (B=%d, %d tokens per "
                      "sequence, H=32, d=128)" % (B, K),
            "value": 1e3 / pair, "unit": "steps/s", "step_ms": pair, "verify_ms": vt, "accept_ms": at,
            "tokens_per_s": B * K / (pair * 1e-3), "sequences_accepting": n_acc,
            "roofline": {"bound": "hbm", "kernel": "decode_tokens_kernel (verify + accept)",
                         "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": _round_traffic(B, K), "bytes_per_step": v_bytes + a_bytes}}


def bench_decode_tokens(B, K, dev, steps=50):
    """Multi-token decode: K tokens per sequence per call, the state read and
    written once per call (kda_decode_tokens without a history), B=256; one
    event pair around ``steps`` back-to-back calls.  Against single-token
    decode the state traffic per token drops K-fold."""
    from gated_delta_rule_76_amd import inputs, kda
    spec = inputs.WORKLOADS["decode_b256"]
    H, D = spec["H"], spec["D"]
    sets = []
    for i in range(N_SETS):
        d = inputs.decode_inputs(B * K, H, D, 1, torch.bfloat16, spec["decay"], spec["s_std"], seed=i,
                                 device=dev)
        sets.append({key: d[key][0].reshape((B, K) + tuple(d[key].shape[2:])).contiguous()
                     for key in ("q", "k", "v", "alpha", "beta")})
    S = inputs.state(B, H, D, spec["s_std"], seed=0, device=dev)
    o = torch.empty((B, K, H, D), dtype=torch.float32, device=dev)
    run = lambda t: kda.decode_tokens(t["q"], t["k"], t["v"], t["alpha"], t["beta"], S, out=o)
    for i in range(5):
        run(sets[i % N_SETS])
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record()
    for i in range(steps):
        run(sets[i % N_SETS])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = B * H * (2 * D * D * 4 + K * (768 + 512 + 4 + 512))
    gbs = nbytes / (ms * 1e-3) / 1e9
    t = _traffic("decode_tokens_kernel", "decode_tokens_b%d_k%d" % (B, K), DECODE_TOKENS_TRAFFIC_SUMMARY % (B, K),
                 DECODE_SOURCE)
    return {"metric": "multi-token decode tokens/s (B=%d, %d tokens per sequence per call, H=32, d=128)" % (B, K),
            "value": B * K / (ms * 1e-3), "unit": "tokens/s", "call_ms": ms,
            "roofline": {"bound": "hbm", "kernel": "decode_tokens_kernel (advance)", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": t,
                         "bytes_per_call": nbytes}}


def bench_verify_fused(B, K, dev, steps=50):
    """Verification rounds in one pass over the state each: every call
    accepts the previous round's seeded accepted counts (the same counts as
    bench_verify) and verifies the next round's tokens (kda_accept_verify_tokens).
    One event pair around ``steps`` back-to-back rounds."""
    from gated_delta_rule_76_amd import inputs, kda
    spec = inputs.WORKLOADS["decode_b256"]
    H, D = spec["H"], spec["D"]
    sets = []
    for i in range(N_SETS):
        d = inputs.decode_inputs(B * K, H, D, 1, torch.bfloat16, spec["decay"], spec["s_std"], seed=i,
                                 device=dev)
        sets.append({key: d[key][0].reshape((B, K) + tuple(d[key].shape[2:])).contiguous()
                     for key in ("q", "k", "v", "alpha", "beta")})
    S = inputs.state(B, H, D, spec["s_std"], seed=0, device=dev)
    o = torch.empty((B, K, H, D), dtype=torch.float32, device=dev)
    g = torch.Generator(device="cpu")
    g.manual_seed(0)
    accepted = torch.randint(0, K + 1, (B,), generator=g, dtype=torch.int32).to(dev)
    keys = ("q", "k", "v", "alpha", "beta")
    # one prepared round per (previous set, this set): the loop makes only the C calls
    calls = [kda.AcceptVerifyCall(tuple(sets[(i + N_SETS - 1) % N_SETS][key] for key in keys), accepted,
                                  *(sets[i][key] for key in keys), S, out=o) for i in range(N_SETS)]

    def rnd(i):
        calls[i % N_SETS].run()
    for i in range(5):
        rnd(i)
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record()
    for i in range(steps):
        rnd(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    n_acc = int((accepted > 0).sum())
    state = D * D * 4
    # the state read once and, for an accepting sequence, written once; the
    # accepted tokens' inputs (all k counted) and this round's inputs and outputs
    nbytes = B * H * (state + K * (768 + 512 + 4 + 512)) + n_acc * H * (state + K * (768 + 512 + 4))
    gbs = nbytes / (ms * 1e-3) / 1e9
    t = _traffic("decode_tokens_kernel", "verify_fused_b%d_k%d" % (B, K), VERIFY_FUSED_TRAFFIC_SUMMARY % (B, K),
                 DECODE_SOURCE)
    return {"metric": "speculative verify steps/s, accept and verify in one pass (B=%d, %d tokens per "
                      "sequence, H=32, d=128)" % (B, K),
            "value": 1e3 / ms, "unit": "steps/s", "step_ms": ms, "tokens_per_s": B * K / (ms * 1e-3),
            "sequences_accepting": n_acc,
            "roofline": {"bound": "hbm", "kernel": "decode_tokens_kernel (accept + verify)", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": t,
                         "bytes_per_step": nbytes}}


def _round_traffic(B, K):
    """Counter bytes of one verify + accept round: the summary averages the
    multi-token kernel's dispatches, verify and accept in equal numbers."""
    t = _traffic("decode_tokens_kernel", "verify_recompute_b%d_k%d" % (B, K),
                 VERIFY_RECOMPUTE_TRAFFIC_SUMMARY % (B, K), DECODE_SOURCE)
    return None if t is None else 2 * t


def bench_backward(name, dev, steps=10, ws_bytes=None):
    """kda_backward over the prefill workload (upstream gradients dO ~ N(0,1),
    dS_T ~ 0.02 N(0,1)); one event pair on the launch stream around ``steps``
    back-to-back calls.  ws_bytes: the workspace (default the recommended
    size; less runs the sequences in pieces)."""
    from gated_delta_rule_76_amd import inputs, kda
    spec = inputs.WORKLOADS[name]
    lens = inputs.workload_lengths(spec, seed=0)
    H, D = spec["H"], spec["D"]
    d = inputs.prefill_inputs(lens, H, D, torch.bfloat16, spec["decay"], spec["s0_std"], seed=0, device=dev)
    T = sum(lens)
    dO, dST = inputs.grad_inputs(T, H, D, len(lens), seed=0, device=dev)
    cu = d["cu_seqlens"] if len(lens) > 1 else None
    if ws_bytes is None:
        ws_bytes = kda.backward_workspace_size(len(lens), T, H, D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    run = lambda: kda.backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dO, d["S0"], dST, cu,
                               workspace=ws)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    gbs = T * H * backward_bytes() / (ms * 1e-3) / 1e9
    # counter bytes of one call (both kernels), for the recommended workspace only
    traffic = None
    if ws_bytes == kda.backward_workspace_size(len(lens), T, H, D):
        parts = [_traffic(kn, name, BACKWARD_TRAFFIC_SUMMARY, BACKWARD_SOURCE)
                 for kn in ("bwd_kernel", "bwd_reduce_kernel")]
        traffic = None if None in parts else sum(parts)
    return {"metric": "KDA backward tokens/s/layer (%s)" % name, "value": T / (ms * 1e-3),
            "unit": "tokens/s/layer", "ms_per_step": ms, "workspace_bytes": int(ws.numel()),
            "roofline": {"bound": "hbm", "kernel": "bwd_kernel + bwd_reduce_kernel", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": traffic, "bytes_per_token_head": backward_bytes()}}


def verify_summary(vf):
    B, K, H = vf["B"], vf["K"], vf["H"]
    gbs = B * H * verify_bytes(K) / (vf["verify_ms"] * 1e-3) / 1e9
    return {"metric": "speculative verify steps/s (B=%d, %d tokens per sequence, H=32, d=128)" % (B, K),
            "value": 1e3 / vf["step_ms"], "unit": "steps/s", "step_ms": vf["step_ms"],
            "verify_ms": vf["verify_ms"], "commit_ms": vf["commit_ms"],
            "tokens_per_s": B * K / (vf["verify_ms"] * 1e-3),
            "roofline": {"bound": "hbm", "kernel": "decode_tokens_kernel", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": _traffic("decode_tokens_kernel", "verify_b%d_k%d" % (B, K),
                                             VERIFY_TRAFFIC_SUMMARY % (B, K), DECODE_SOURCE),
                         "bytes_per_seq_head": verify_bytes(K)},
            "commit": {"sequences_committed": vf["committed_seqs"],
                       "achieved_gbs": vf["committed_seqs"] * H * 2 * 128 * 128 * 4 / (vf["commit_ms"] * 1e-3) / 1e9}}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, one process per group of heads
# (or of (sequence, head) pairs for decode) on the host cores.  Runs before
# anything touches the GPU (the worker processes are forked).
# ---------------------------------------------------------------------------
_CPU_INPUTS = {}


def _cpu_prefill_worker(heads):
    from threadpoolctl import threadpool_limits

    from oracle import gdn_recurrent, kda_recurrent
    from oracle.prologue import recurrent_from_preact
    a = _CPU_INPUTS
    run = gdn_recurrent if a["gate"] == "head" else kda_recurrent
    if a["form"] == "preact":
        run = recurrent_from_preact
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for _ in range(a["passes"]):
            run(a["q"][:, heads], a["k"][:, heads], a["v"][:, heads], a["alpha"][:, heads],
                          a["beta"][:, heads], None if a["S0"] is None else a["S0"][:, heads],
                          cu_seqlens=a["cu"])
        return time.perf_counter() - t0


def _cpu_decode_worker(pairs):
    from threadpoolctl import threadpool_limits

    from oracle import gdn_decode_step, kda_decode_step
    a = _CPU_INPUTS
    step = gdn_decode_step if a["gate"] == "head" else kda_decode_step
    with threadpool_limits(limits=1):
        S = a["S"][pairs]
        t0 = time.perf_counter()
        for s in range(a["steps"]):
            _, S = step(a["q"][s][pairs], a["k"][s][pairs], a["v"][s][pairs],
                                   a["alpha"][s][pairs], a["beta"][s][pairs], S)
        return time.perf_counter() - t0


def _cpu_verify_worker(seqs):
    from threadpoolctl import threadpool_limits

    from oracle import speculative
    a = _CPU_INPUTS
    K = a["K"]
    rows = (seqs[:, None] * K + np.arange(K)[None, :]).ravel()
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        speculative.decode_tokens(a["q"][rows], a["k"][rows], a["v"][rows], a["alpha"][rows],
                                  a["beta"][rows], a["S"][seqs], K)
        return time.perf_counter() - t0


def _cpu_backward_worker(heads):
    from threadpoolctl import threadpool_limits

    from oracle.backward import kda_backward
    a = _CPU_INPUTS
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        kda_backward(a["q"][:, heads], a["k"][:, heads], a["v"][:, heads], a["alpha"][:, heads],
                     a["beta"][:, heads], a["dO"][:, heads], None, a["dST"][:, heads])
        return time.perf_counter() - t0


def _pool_map(fn, n_items):
    import multiprocessing as mp
    workers = max(1, min(16, os.cpu_count() or 1, n_items))
    groups = [g for g in np.array_split(np.arange(n_items), workers) if len(g)]
    with mp.get_context("fork").Pool(len(groups)) as pool:
        t0 = time.perf_counter()
        busy = pool.map(fn, groups)
        wall = time.perf_counter() - t0
    return wall, sum(busy), len(groups)


def oracle_prefill_rate(workload, max_tokens=None, passes=1, gate="channel", form="final"):
    """Oracle tokens/s/layer over ``workload`` (or its first ``max_tokens``
    tokens when the sequence is longer), all heads, ``passes`` repetitions."""
    from gated_delta_rule_76_amd import inputs
    spec = inputs.WORKLOADS[workload]
    lengths = inputs.workload_lengths(spec, seed=0)
    prefix = max_tokens is not None and sum(lengths) > max_tokens
    if prefix:
        lengths = [max_tokens]
    d = inputs.prefill_inputs(lengths, spec["H"], spec["D"], torch.bfloat16, spec["decay"],
                              None if prefix else spec["s0_std"], seed=0, device="cpu", gate=gate,
                              form=form)
    _CPU_INPUTS["gate"] = gate
    _CPU_INPUTS["form"] = form
    _CPU_INPUTS.update({k: d[k].double().numpy() for k in ("q", "k", "v", "alpha", "beta")})
    _CPU_INPUTS["S0"] = None if d["S0"] is None else d["S0"].double().numpy()
    _CPU_INPUTS["cu"] = d["cu_seqlens"].numpy()
    _CPU_INPUTS["passes"] = passes
    T = sum(lengths)
    wall, busy, cores = _pool_map(_cpu_prefill_worker, spec["H"])
    _CPU_INPUTS.clear()
    what = (f"the first {T} tokens of {workload}" if prefix else f"the whole {workload} workload")
    if gate == "head":
        what += " with one alpha per token and head"
    if form == "preact":
        what += " from pre-activations"
    return {"value": passes * T / wall, "unit": "tokens/s/layer", "cores": cores, "kind": "oracle",
            "sample": f"{what} ({T} tokens x {spec['H']} heads, d={spec['D']}"
                      f"{', x%d passes' % passes if passes > 1 else ''}), numpy fp64 token-by-token "
                      f"recurrence, {cores} processes over head groups ({wall:.2f} s wall, "
                      f"{busy:.1f} s CPU)"}


def oracle_decode_rate(B=256, steps=100, gate="channel"):
    """Oracle steps/s: ``steps`` decode steps of B sequences x 32 heads, d=128."""
    from gated_delta_rule_76_amd import inputs
    spec = inputs.WORKLOADS["decode_b256"]
    H, D = spec["H"], spec["D"]
    d = inputs.decode_inputs(B, H, D, steps, torch.bfloat16, spec["decay"], spec["s_std"], seed=0,
                             device="cpu", gate=gate)
    n = B * H
    _CPU_INPUTS["gate"] = gate
    _CPU_INPUTS["S"] = d["S"].double().numpy().reshape(n, 1, D, D)
    for k in ("q", "k", "v"):
        _CPU_INPUTS[k] = d[k].double().numpy().reshape(steps, n, 1, D)
    _CPU_INPUTS["alpha"] = d["alpha"].double().numpy().reshape((steps, n, 1) + ((D,) if gate == "channel" else ()))
    _CPU_INPUTS["beta"] = d["beta"].double().numpy().reshape(steps, n, 1)
    _CPU_INPUTS["steps"] = steps
    wall, busy, cores = _pool_map(_cpu_decode_worker, n)
    _CPU_INPUTS.clear()
    return {"value": steps / wall, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"{steps} decode steps, B={B} H={H} d={D}"
                      f"{', one alpha per head' if gate == 'head' else ''}, numpy fp64, {cores} processes "
                      f"over (sequence, head) groups ({wall:.2f} s wall, {busy:.1f} s CPU)"}


def oracle_verify_rate(B=256, K=2):
    """Oracle steps/s of speculative verification: K tokens for each of B
    sequences x 32 heads with every intermediate state kept."""
    from gated_delta_rule_76_amd import inputs
    spec = inputs.WORKLOADS["decode_b256"]
    H, D = spec["H"], spec["D"]
    d = inputs.decode_inputs(B * K, H, D, 1, torch.bfloat16, spec["decay"], spec["s_std"], seed=0,
                             device="cpu")
    for key in ("q", "k", "v", "alpha", "beta"):
        _CPU_INPUTS[key] = d[key][0].double().numpy()
    _CPU_INPUTS["S"] = d["S"][:B].double().numpy()
    _CPU_INPUTS["K"] = K
    wall, busy, cores = _pool_map(_cpu_verify_worker, B)
    _CPU_INPUTS.clear()
    return {"value": 1.0 / wall, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"one verify step, B={B} sequences x {K} tokens, H={H} d={D}, states kept, "
                      f"numpy fp64, {cores} processes over sequence groups ({wall:.2f} s wall, "
                      f"{busy:.1f} s CPU)"}


def oracle_backward_rate():
    """Oracle tokens/s/layer of the backward pass over the prefill_4k workload."""
    from gated_delta_rule_76_amd import inputs
    spec = inputs.WORKLOADS["prefill_4k"]
    T, H, D = spec["lengths"][0], spec["H"], spec["D"]
    d = inputs.prefill_inputs([T], H, D, torch.bfloat16, spec["decay"], None, seed=0, device="cpu")
    dO, dST = inputs.grad_inputs(T, H, D, 1, seed=0, device="cpu")
    _CPU_INPUTS.update({k: d[k].double().numpy() for k in ("q", "k", "v", "alpha", "beta")})
    _CPU_INPUTS["dO"], _CPU_INPUTS["dST"] = dO.double().numpy(), dST.double().numpy()
    wall, busy, cores = _pool_map(_cpu_backward_worker, H)
    _CPU_INPUTS.clear()
    return {"value": T / wall, "unit": "tokens/s/layer", "cores": cores, "kind": "oracle",
            "sample": f"backward of the whole prefill_4k workload ({T} tokens x {H} heads, d={D}), numpy "
                      f"fp64, {cores} processes over head groups ({wall:.2f} s wall, {busy:.1f} s CPU)"}


def cpu_baseline():
    return oracle_prefill_rate("prefill_4k", passes=3)


def oracle_rates():
    """Every workload's oracle rate; the 2^20-token sequence is timed on its
    first 65,536 tokens and extrapolated linearly (the per-token cost of the
    recurrence does not depend on the position)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    out = {"host_cpus": os.cpu_count(), "cpu_model": model,
           "prefill_4k": oracle_prefill_rate("prefill_4k", passes=3),
           "varlen_8seq": oracle_prefill_rate("varlen_8seq"),
           "decode_b256": oracle_decode_rate(256, 100)}
    lg = oracle_prefill_rate("long_1m", max_tokens=65536)
    lg["extrapolated_seconds_for_2^20_tokens"] = (1 << 20) / lg["value"]
    out["long_1m"] = lg
    out["prefill_4k_scalar_gate"] = oracle_prefill_rate("prefill_4k", passes=3, gate="head")
    out["decode_b256_scalar_gate"] = oracle_decode_rate(256, 100, gate="head")
    out["prefill_4k_preact"] = oracle_prefill_rate("prefill_4k", passes=3, form="preact")
    out["verify_b256_k2"] = oracle_verify_rate(256, 2)
    out["backward_prefill_4k"] = oracle_backward_rate()
    return out


def _traffic(kernel, workload, summary=None, source=None):
    """HBM bytes per launch of ``kernel`` from a committed counter summary
    (the prefill one unless ``summary`` / ``source`` name another), or None
    when it is missing or was taken on other kernel source."""
    summary = TRAFFIC_SUMMARY if summary is None else summary
    source = KERNEL_SOURCE if source is None else source
    try:
        with open(summary) as f:
            t = json.load(f)
        with open(source, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(kernel)
    if t.get("source_sha256") != sha or t.get("workload") != workload or k is None:
        return None
    return k["fetch_bytes"] + k["write_bytes"]


def _mfma_issued(workload, suffix=""):
    """Issued matrix-core flops per prefill call from the committed counter
    summary (of the variant ``suffix`` names), per kernel, or None when it is
    missing or was taken on other kernel source."""
    try:
        with open(_variant_path(MFMA_SUMMARY, suffix)) as f:
            t = json.load(f)
        with open(KERNEL_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != sha or t.get("workload") != workload + suffix:
        return None
    return {k: v["issued_flop"] for k, v in t.get("kernels", {}).items()}


def prefill_summary(pf, gate, workload=None, form="final"):
    """Rate, the dominant kernel's roofline and the matrix-core figures of
    one bench_prefill result.

    ``roofline`` follows the layer's algorithmic bytes: 1,796 bytes per token
    and head (q, k, v, alpha, beta read, o written; 1,288 with one alpha per
    head) times the token-heads of one call, over the dominant kernel's
    event-timed duration.  ``kernels`` gives each kernel's time and the
    bytes it moves itself, its workspace record included.  ``mfma`` gives the
    issued matrix-core rate (counters) and the useful one (139,264 flop per
    token and head) over the call, and the call's rate against the lower of
    the HBM and matrix-core ceilings."""
    th = pf["total_tokens"] * pf["H"]
    kb = kernel_bytes(pf["D"], gate)
    times = {"chunk_local_kernel": pf["phases_ms"]["chunk_local"],
             "chunk_state_kernel": pf["phases_ms"]["state_pass"]}
    dom = max(times, key=times.get)
    own = {k: th * kb[k] / (times[k] * 1e-3) / 1e9 for k in times}
    lb = layer_bytes(gate)
    alg = th * lb / (times[dom] * 1e-3) / 1e9
    layer_gbs = th * lb / (pf["ms"] * 1e-3) / 1e9
    value = pf["total_tokens"] / (pf["ms"] * 1e-3)
    suffix = VARIANT_SUFFIX.get((gate, form))
    issued = _mfma_issued(workload, suffix) if workload is not None and suffix is not None else None
    hbm_ceiling = HBM_PEAK_GBS * 1e9 / (lb * pf["H"])
    mf = {"peak_tflops": MFMA_PEAK_TFLOPS, "useful_flop_per_token_head": USEFUL_FLOP_PER_TOKEN_HEAD,
          "useful_tflops": th * USEFUL_FLOP_PER_TOKEN_HEAD / (pf["ms"] * 1e-3) / 1e12,
          "issued_tflops": None, "issued_frac": None, "issued_flop_per_token_head": None,
          "counters": None}
    mf["useful_frac"] = mf["useful_tflops"] / MFMA_PEAK_TFLOPS
    ceiling = hbm_ceiling
    if issued is not None and all(k in issued for k in times):
        per_call = sum(issued[k] for k in times)
        mf["issued_flop_per_token_head"] = per_call / th
        mf["issued_tflops"] = per_call / (pf["ms"] * 1e-3) / 1e12
        mf["issued_frac"] = mf["issued_tflops"] / MFMA_PEAK_TFLOPS
        mf["counters"] = os.path.relpath(_variant_path(MFMA_SUMMARY, suffix), ROOT)
        ceiling = min(hbm_ceiling, MFMA_PEAK_TFLOPS * 1e12 / (per_call / th * pf["H"]))
    mf["ceiling_tokens_per_s"] = ceiling
    mf["frac_of_ceiling"] = value / ceiling
    return {"value": value, "unit": "tokens/s/layer",
            "ms_per_step": pf["ms"],
            "roofline": {"bound": "hbm", "kernel": dom, "achieved": alg, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": alg / HBM_PEAK_GBS, "traffic": None,
                         "launch_ms": times[dom], "bytes_per_token_head": lb},
            "kernels": {k: {"ms": times[k], "own_bytes_per_token_head": kb[k], "own_gbs": own[k]}
                        for k in times},
            "layer_roofline": {"bound": "hbm", "bytes_per_token_head": lb, "achieved": layer_gbs,
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": layer_gbs / HBM_PEAK_GBS},
            "mfma": mf}


def decode_summary(dc, gate, form="final"):
    gbs = dc["B"] * dc["H"] * decode_bytes(gate) / (dc["ms_per_step"] * 1e-3) / 1e9
    # (the counter summary covers the per-channel decode kernel on activated inputs)
    traffic = (_traffic("decode_kernel", "decode_b%d" % dc["B"], DECODE_TRAFFIC_SUMMARY % dc["B"],
                        DECODE_SOURCE)
               if gate == "channel" and form == "final" else None)
    kind = ("KDA" if gate == "channel" else "scalar-gate") + (" pre-activation" if form == "preact" else "")
    return {"metric": "%s decode steps/s (B=%d, H=32, d=128)" % (kind, dc["B"]),
            "value": 1e3 / dc["ms_per_step"], "unit": "steps/s", "ms_per_step": dc["ms_per_step"],
            "roofline": {"bound": "hbm", "kernel": "decode_kernel", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": traffic, "bytes_per_head_step": decode_bytes(gate)},
            "state_rmw_gbs": dc["state_rmw_gbs"]}


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer shards by "
              "(sequence, head) with no communication between GPUs, so one GPU's rate is the unit)",
              file=sys.stderr)
        sys.exit(2)
    if args.oracle_rates:
        print(json.dumps(oracle_rates()), flush=True)
        return
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        # float64, which nothing else in this program uses, so the copy's
        # dispatches are easy to pick out of a counter trace
        src = torch.ones(COPY_BYTES // 8, dtype=torch.float64, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 0.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if args.only == "backward":
        print("[bench] backward only", file=sys.stderr, flush=True)
        print(json.dumps({"backward": bench_backward("prefill_4k", dev)}), flush=True)
        return
    if args.only == "verify":
        print("[bench] speculative verify only", file=sys.stderr, flush=True)
        print(json.dumps({"verify": verify_summary(bench_verify(args.decode_batch, 2, dev))}), flush=True)
        return
    if args.only in ("prefill_head", "prefill_preact"):
        gate, form = ("head", "final") if args.only == "prefill_head" else ("channel", "preact")
        print(f"[bench] {args.only} only", file=sys.stderr, flush=True)
        pv = bench_prefill(args.workload, args.steps, args.warmup, dev, gate=gate, form=form)
        print(json.dumps({args.only: prefill_summary(pv, gate, args.workload, form)}), flush=True)
        return
    if args.only == "verify_fused":
        print("[bench] speculative verify, accept and verify in one pass, only", file=sys.stderr, flush=True)
        print(json.dumps({"verify_fused": bench_verify_fused(args.decode_batch, 2, dev)}), flush=True)
        return
    if args.only == "decode_tokens":
        print("[bench] multi-token decode only", file=sys.stderr, flush=True)
        print(json.dumps({"decode_tokens_k4": bench_decode_tokens(args.decode_batch, 4, dev)}), flush=True)
        return
    if args.only == "verify_recompute":
        print("[bench] speculative verify by recomputation only", file=sys.stderr, flush=True)
        print(json.dumps({"verify_recompute": bench_verify_recompute(args.decode_batch, 2, dev)}), flush=True)
        return
    print(f"[bench] prefill {args.workload}: warmup {args.warmup}, steps {args.steps}", file=sys.stderr,
          flush=True)
    pf = bench_prefill(args.workload, args.steps, args.warmup, dev)
    ps = prefill_summary(pf, "channel", args.workload)
    dom = ps["roofline"]["kernel"]
    ps["roofline"]["traffic"] = _traffic(dom, args.workload)
    out = {
        "metric": "KDA prefill tokens/s/layer (H=32, d=128)",
        "value": ps["value"],
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOAD_TEXT[args.workload]}, bf16 q/k/v, "
                               "fp32 alpha/beta/state/o, chunk 64",
                   "total_tokens": pf["total_tokens"], "heads": pf["H"], "head_dim": pf["D"]},
        "roofline": ps["roofline"],
        "kernels": ps["kernels"],
        "layer_roofline": ps["layer_roofline"],
        "mfma": ps["mfma"],
        "call_ms": pf["call_ms"],
        "stalled_calls": pf["stalled_calls"],
    }
    if args.bounded_workspace_mib:
        print(f"[bench] prefill with a {args.bounded_workspace_mib} MiB workspace", file=sys.stderr, flush=True)
        out["bounded_workspace"] = bench_bounded(args.workload, args.steps, args.warmup, dev,
                                                 args.bounded_workspace_mib << 20)
    if not args.no_decode:
        print("[bench] decode", file=sys.stderr, flush=True)
        out["decode"] = decode_summary(bench_decode(args.decode_batch, dev), "channel")
        if not args.no_variants:
            out["decode"]["context_growth"] = bench_decode_context(args.decode_batch, dev)
        if not args.no_variants and args.decode_large_batch:
            print(f"[bench] decode at B={args.decode_large_batch}", file=sys.stderr, flush=True)
            out["decode_large"] = decode_summary(bench_decode(args.decode_large_batch, dev), "channel")
    if not args.no_variants:
        # The scalar-gate (Gated DeltaNet) form on the same shapes.
        print("[bench] scalar gate", file=sys.stderr, flush=True)
        pv = bench_prefill(args.workload, args.steps, args.warmup, dev, gate="head")
        sg = {"prefill": prefill_summary(pv, "head", args.workload)}
        sg["prefill"]["roofline"]["traffic"] = _traffic(sg["prefill"]["roofline"]["kernel"], args.workload + "_head",
                                                        _variant_path(TRAFFIC_SUMMARY, "_head"))
        sg["prefill"]["metric"] = "scalar-gate prefill tokens/s/layer (H=32, d=128)"
        sg["prefill"]["call_ms"] = pv["call_ms"]
        sg["prefill"]["stalled_calls"] = pv["stalled_calls"]
        if not args.no_decode:
            sg["decode"] = decode_summary(bench_decode(args.decode_batch, dev, gate="head"), "head")
        out["scalar_gate"] = sg
        # Pre-activation inputs (gate and normalisation prologue in the load
        # stage); the bytes moved are the same as for activated inputs.
        print("[bench] pre-activation inputs", file=sys.stderr, flush=True)
        pp = bench_prefill(args.workload, args.steps, args.warmup, dev, form="preact")
        pa = {"prefill": prefill_summary(pp, "channel", args.workload, "preact")}
        pa["prefill"]["roofline"]["traffic"] = _traffic(pa["prefill"]["roofline"]["kernel"],
                                                        args.workload + "_preact",
                                                        _variant_path(TRAFFIC_SUMMARY, "_preact"))
        pa["prefill"]["metric"] = "KDA prefill from pre-activations, tokens/s/layer (H=32, d=128)"
        pa["prefill"]["call_ms"] = pp["call_ms"]
        pa["prefill"]["stalled_calls"] = pp["stalled_calls"]
        if not args.no_decode:
            pa["decode"] = decode_summary(bench_decode(args.decode_batch, dev, form="preact"), "channel",
                                          "preact")
        out["preact"] = pa
        if not args.no_decode:
            print("[bench] speculative verify", file=sys.stderr, flush=True)
            out["verify"] = verify_summary(bench_verify(args.decode_batch, 2, dev))
            out["verify_recompute"] = bench_verify_recompute(args.decode_batch, 2, dev)
            out["verify_fused"] = bench_verify_fused(args.decode_batch, 2, dev)
            out["decode_tokens_k4"] = bench_decode_tokens(args.decode_batch, 4, dev)
        print("[bench] backward", file=sys.stderr, flush=True)
        out["backward"] = bench_backward(args.workload if args.workload == "prefill_4k" else "prefill_4k", dev)
        if args.bounded_backward_mib:
            out["backward"]["bounded_workspace"] = bench_backward(
                "prefill_4k", dev, ws_bytes=args.bounded_backward_mib << 20)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
