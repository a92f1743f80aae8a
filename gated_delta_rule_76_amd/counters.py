"""HBM traffic of the prefill or decode kernels from two rocprofv3 counter
runs of bench.py.

    rocprofv3 --pmc FETCH_SIZE -d DIR_F -o f --output-format csv -- \\
        python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-decode --no-variants \\
        --calibrate-copy
    rocprofv3 --pmc WRITE_SIZE -d DIR_W -o w --output-format csv -- \\
        python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-decode --no-variants \\
        --calibrate-copy
    python -m gated_delta_rule_76_amd.counters DIR_F/f_counter_collection.csv \\
        DIR_W/w_counter_collection.csv --workload prefill_4k > profiles/traffic_prefill_4k.json

(--no-variants: only the per-channel, activated-input kernels run, which
the summary matches by name), and for the decode step (bench.py without
--no-decode, with --no-variants so that only the per-channel decode kernel
runs):

    python -m gated_delta_rule_76_amd.counters F.csv W.csv --target decode \\
        --workload decode_b256 > profiles/traffic_decode_b256.json

The backward and the speculative verification leg alone (bench.py --only
backward / --only verify, each with --calibrate-copy):

    python -m gated_delta_rule_76_amd.counters F.csv W.csv --target backward \\
        --workload prefill_4k > profiles/traffic_backward_4k.json
    python -m gated_delta_rule_76_amd.counters F.csv W.csv --target decode \\
        --workload verify_b256_k2 > profiles/traffic_verify_b256_k2.json

The multi-token decode leg (bench.py --only decode_tokens --calibrate-copy):

    python -m gated_delta_rule_76_amd.counters F.csv W.csv --target decode \\
        --workload decode_tokens_b256_k4 > profiles/traffic_decode_tokens_b256_k4.json

FETCH_SIZE and WRITE_SIZE are read per dispatch (KiB).  Each is scaled by
the factor that maps the same counter of a plain elementwise float64 copy
of 256 MiB (the --calibrate-copy kernel, which reads and writes exactly
that, in 16-byte accesses like the library's kernels) to its true size.
The summary records the sha256 of the kernel source it was taken on;
bench.py reports the traffic only while the source matches.

Matrix-core work of the prefill kernels, from one counter run:

    rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 -d DIR_M -o m \
        --output-format csv -- python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline \
        --no-decode --no-variants
    python -m gated_delta_rule_76_amd.counters --mfma DIR_M/m_counter_collection.csv \
        --workload prefill_4k > profiles/mfma_prefill_4k.json

Each MOPS unit is 512 floating-point operations (one per multiply and one
per add of the matrix product); the summary gives the issued flops per
dispatch of each kernel, which bench.py divides by the event-timed call.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_76_amd", "csrc")
COPY_BYTES = 256 << 20
# kernel source and kernel names per target ("decode_kernel" is not a
# substring of "decode_tokens_kernel")
TARGETS = {
    "prefill": ("kda_prefill.hip", ("chunk_local_kernel", "chunk_state_kernel")),
    "decode": ("kda_decode.hip", ("decode_kernel", "decode_tokens_kernel", "commit_kernel")),
    "backward": ("kda_backward.hip", ("bwd_kernel", "bwd_reduce_kernel")),
}


def _per_kernel(path, counter, kernels):
    vals = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = None
            for k in kernels:
                if k in name:
                    key = k
            low = name.lower()
            if key is None and "elementwise" in low and "add" in low and "double" in low:
                key = "copy"
            if key is not None:
                vals[key].append(float(r["Counter_Value"]) * 1024.0)
    return vals


def summarize(fetch_csv, write_csv, workload, target="prefill"):
    source, kernels = TARGETS[target]
    fv = _per_kernel(fetch_csv, "FETCH_SIZE", kernels)
    wv = _per_kernel(write_csv, "WRITE_SIZE", kernels)
    # the copy runs three times; take the median dispatch
    cf = sorted(fv["copy"])[len(fv["copy"]) // 2]
    cw = sorted(wv["copy"])[len(wv["copy"]) // 2]
    f_fetch, f_write = COPY_BYTES / cf, COPY_BYTES / cw
    with open(os.path.join(CSRC, source), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    out = {"workload": workload, "source_sha256": sha,
           "calibration": {"copy_bytes": COPY_BYTES, "copy_fetch_counter_bytes": cf,
                           "copy_write_counter_bytes": cw, "fetch_factor": f_fetch,
                           "write_factor": f_write},
           "kernels": {}}
    for k in kernels:
        if fv.get(k) and wv.get(k):
            fr = sum(fv[k]) / len(fv[k])
            wr = sum(wv[k]) / len(wv[k])
            out["kernels"][k] = {"dispatches": len(fv[k]), "fetch_counter_bytes": fr,
                                 "write_counter_bytes": wr, "fetch_bytes": fr * f_fetch,
                                 "write_bytes": wr * f_write}
    return out


FLOP_PER_MOP = 512


def _raw_per_kernel(path, counter, kernels):
    vals = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = None
            for k in kernels:
                if k in r["Kernel_Name"]:
                    key = k
            if key is not None:
                vals[key].append(float(r["Counter_Value"]))
    return vals


def summarize_mfma(csv_path, workload, target="prefill"):
    source, kernels = TARGETS[target]
    bf = _raw_per_kernel(csv_path, "SQ_INSTS_VALU_MFMA_MOPS_BF16", kernels)
    f32 = _raw_per_kernel(csv_path, "SQ_INSTS_VALU_MFMA_MOPS_F32", kernels)
    with open(os.path.join(CSRC, source), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    out = {"workload": workload, "source_sha256": sha, "flop_per_mop": FLOP_PER_MOP, "kernels": {}}
    for k in kernels:
        if bf.get(k):
            b = sum(bf[k]) / len(bf[k])
            x = sum(f32[k]) / len(f32[k]) if f32.get(k) else 0.0
            out["kernels"][k] = {"dispatches": len(bf[k]), "mops_bf16": b, "mops_f32": x,
                                 "issued_flop": (b + x) * FLOP_PER_MOP}
    return out


def main():
    p = argparse.ArgumentParser()
    p.add_argument("csv", nargs="+", help="FETCH_SIZE and WRITE_SIZE csv files, or with --mfma the "
                                          "MFMA counter csv")
    p.add_argument("--mfma", action="store_true")
    p.add_argument("--workload", default="prefill_4k")
    p.add_argument("--target", default="prefill", choices=sorted(TARGETS))
    a = p.parse_args()
    if a.mfma:
        print(json.dumps(summarize_mfma(a.csv[0], a.workload, a.target), indent=1))
    else:
        print(json.dumps(summarize(a.csv[0], a.csv[1], a.workload, a.target), indent=1))


if __name__ == "__main__":
    main()
