"""Benchmark of the KDA layer on one MI355X: prefill tokens/s/layer and decode steps/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-decode]

A step is one kda_prefill call (schedule, chunk-local matrices, state pass)
over one batch of the prefill workload (default prefill_4k: B=1, H=32,
T=4096, d=128, bf16 q/k/v, fp32 alpha/beta/state/o, seeded synthetic
inputs resident in HBM).  Three input sets are rotated so that consecutive
steps do not find their ~235 MB working set in the 256 MB Infinity Cache.
Prints one JSON line with the prefill rate as ``value``, the roofline of the
dominant kernel, the decode rate of the decode workload (B=256, H=32,
d=128, 100 in-place steps), and the fp64 CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores

# Algorithmic bytes per token and head (d = 128).
#  whole prefill: q,k,v bf16 (768) + alpha fp32 (512) + beta (4) + o fp32 (512)
#  state pass:    q,k,v (768) + alpha (512) + T,M chunk matrices (512) + o (512)
#  chunk-local:   q,k (512) + alpha (512) + beta (4) + T,M written (512)
BYTES_PREFILL = 768 + 512 + 4 + 512
BYTES_STATE_PASS = 768 + 512 + 512 + 512
BYTES_CHUNK_LOCAL = 512 + 512 + 4 + 512
# Decode per (sequence, head) and step: state read + write, q,k,v, alpha, beta, o.
BYTES_DECODE = 2 * 128 * 128 * 4 + 768 + 512 + 4 + 512


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="prefill_4k",
                   choices=["prefill_4k", "varlen_8seq", "long_1m"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--decode-batch", type=int, default=256)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 256 MiB device copy (a known-size kernel for "
                        "scaling hardware byte counters)")
    return p.parse_args()


def _events():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def bench_prefill(name, steps, warmup, dev):
    from gated_delta_rule_76_amd import inputs, kda
    spec = inputs.WORKLOADS[name]
    lens = inputs.workload_lengths(spec, seed=0)
    H, D = spec["H"], spec["D"]
    n_sets = 3 if sum(lens) <= 65536 else 1
    calls = []
    for s in range(n_sets):
        d = inputs.prefill_inputs(lens, H, D, torch.bfloat16, spec["decay"], spec["s0_std"],
                                  seed=s, device=dev)
        cu = d["cu_seqlens"] if len(lens) > 1 else None
        calls.append(kda.PrefillCall(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], cu))
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
    # Per-phase timing with events on the launch stream (the current stream).
    ph = {"chunk_local": 0.0, "state_pass": 0.0}
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
    for a, b, c in evs:
        ph["chunk_local"] += a.elapsed_time(b) / steps
        ph["state_pass"] += b.elapsed_time(c) / steps
    return {"total_tokens": total, "H": H, "D": D, "ms": ms, "wall_s": wall, "phases_ms": ph,
            "lengths": lens}


def bench_decode(B, steps, warmup, dev):
    from gated_delta_rule_76_amd import inputs, kda
    spec = inputs.WORKLOADS["decode_b256"]
    H, D = spec["H"], spec["D"]
    d = inputs.decode_inputs(B, H, D, spec["steps"], torch.bfloat16, spec["decay"], spec["s_std"],
                             seed=0, device=dev)
    S = d["S"].clone()
    o = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    n = spec["steps"]
    for s in range(warmup):
        kda.decode_step(d["q"][s % n], d["k"][s % n], d["v"][s % n], d["alpha"][s % n],
                        d["beta"][s % n], S, out=o)
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record()
    for s in range(n):
        kda.decode_step(d["q"][s], d["k"][s], d["v"][s], d["alpha"][s], d["beta"][s], S, out=o)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    return {"B": B, "H": H, "D": D, "steps": n, "ms_per_step": ms}


def cpu_baseline():
    """The fp64 oracle on the host, single-threaded, on a bounded sample of
    the prefill_4k workload: all 32 heads, the first 1024 tokens."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from gated_delta_rule_76_amd import inputs
    from oracle import kda_recurrent
    spec = inputs.WORKLOADS["prefill_4k"]
    T = 1024
    d = inputs.token_inputs(T, spec["H"], spec["D"], torch.bfloat16, spec["decay"], seed=0, device="cpu")
    a = {k: v.double().numpy() for k, v in d.items()}
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        kda_recurrent(a["q"], a["k"], a["v"], a["alpha"], a["beta"])
        dt = time.perf_counter() - t0
    return {"value": T / dt, "unit": "tokens/s/layer", "cores": 1, "kind": "oracle",
            "sample": f"prefill_4k inputs, all {spec['H']} heads, first {T} tokens, numpy fp64, "
                      f"one thread ({dt:.2f} s)"}


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the layer shards by head/sequence with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] prefill {args.workload}: warmup {args.warmup}, steps {args.steps}", file=sys.stderr,
          flush=True)
    pf = bench_prefill(args.workload, args.steps, args.warmup, dev)
    th = pf["total_tokens"] * pf["H"]
    tok_s = pf["total_tokens"] / (pf["ms"] * 1e-3)
    sp_ms = pf["phases_ms"]["state_pass"]
    cl_ms = pf["phases_ms"]["chunk_local"]
    dom, dom_ms, dom_bytes = (("chunk_state_kernel", sp_ms, BYTES_STATE_PASS) if sp_ms >= cl_ms
                              else ("chunk_local_kernel", cl_ms, BYTES_CHUNK_LOCAL))
    achieved = th * dom_bytes / (dom_ms * 1e-3) / 1e9
    out = {
        "metric": "KDA prefill tokens/s/layer (H=32, d=128)",
        "value": tok_s,
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
        "config": {"workload": f"{args.workload}: " + (
            "B=1 H=32 T=4096 d=128" if args.workload == "prefill_4k" else
            "8 seqs, lengths U[1024,16384], H=32 d=128, S0~0.02N" if args.workload == "varlen_8seq" else
            "B=1 H=32 T=1048576 d=128") + ", bf16 q/k/v, fp32 alpha/beta/state/o, chunk 64",
            "total_tokens": pf["total_tokens"], "heads": pf["H"], "head_dim": pf["D"]},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "launch_ms": dom_ms},
        "layer_roofline": {"bound": "hbm", "bytes_per_token_head": BYTES_PREFILL,
                           "achieved": th * BYTES_PREFILL / (pf["ms"] * 1e-3) / 1e9,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": th * BYTES_PREFILL / (pf["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "phases_ms": pf["phases_ms"],
    }
    if not args.no_decode:
        print("[bench] decode", file=sys.stderr, flush=True)
        dc = bench_decode(args.decode_batch, 100, 10, dev)
        gbs = dc["B"] * dc["H"] * BYTES_DECODE / (dc["ms_per_step"] * 1e-3) / 1e9
        out["decode"] = {"metric": "KDA decode steps/s (B=%d, H=32, d=128)" % dc["B"],
                         "value": 1e3 / dc["ms_per_step"], "unit": "steps/s",
                         "ms_per_step": dc["ms_per_step"],
                         "roofline": {"bound": "hbm", "kernel": "decode_kernel", "achieved": gbs,
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": gbs / HBM_PEAK_GBS, "traffic": None}}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
