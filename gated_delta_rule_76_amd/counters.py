"""HBM traffic of the prefill kernels from two rocprofv3 counter runs of bench.py.

    rocprofv3 --pmc FETCH_SIZE -d DIR_F -o f --output-format csv -- \\
        python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-decode --calibrate-copy
    rocprofv3 --pmc WRITE_SIZE -d DIR_W -o w --output-format csv -- \\
        python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-decode --calibrate-copy
    python -m gated_delta_rule_76_amd.counters DIR_F/f_counter_collection.csv \\
        DIR_W/w_counter_collection.csv --workload prefill_4k > profiles/traffic_prefill_4k.json

FETCH_SIZE and WRITE_SIZE are read per dispatch (KiB).  Each is scaled by
the factor that maps the same counter of a plain elementwise float64 copy
of 256 MiB (the --calibrate-copy kernel, which reads and writes exactly
that, in 16-byte accesses like the prefill kernels) to its true size.  The summary records the sha256 of the prefill source it
was taken on; bench.py reports the traffic only while the source matches.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "gated_delta_rule_76_amd", "csrc", "kda_prefill.hip")
COPY_BYTES = 256 << 20
KERNELS = ("chunk_local_kernel", "chunk_state_kernel")


def _per_kernel(path, counter):
    vals = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = None
            for k in KERNELS:
                if k in name:
                    key = k
            low = name.lower()
            if key is None and "elementwise" in low and "add" in low and "double" in low:
                key = "copy"
            if key is not None:
                vals[key].append(float(r["Counter_Value"]) * 1024.0)
    return vals


def summarize(fetch_csv, write_csv, workload):
    fv = _per_kernel(fetch_csv, "FETCH_SIZE")
    wv = _per_kernel(write_csv, "WRITE_SIZE")
    # the copy runs three times; take the median dispatch
    cf = sorted(fv["copy"])[len(fv["copy"]) // 2]
    cw = sorted(wv["copy"])[len(wv["copy"]) // 2]
    f_fetch, f_write = COPY_BYTES / cf, COPY_BYTES / cw
    with open(SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    out = {"workload": workload, "source_sha256": sha,
           "calibration": {"copy_bytes": COPY_BYTES, "copy_fetch_counter_bytes": cf,
                           "copy_write_counter_bytes": cw, "fetch_factor": f_fetch,
                           "write_factor": f_write},
           "kernels": {}}
    for k in KERNELS:
        if fv.get(k) and wv.get(k):
            fr = sum(fv[k]) / len(fv[k])
            wr = sum(wv[k]) / len(wv[k])
            out["kernels"][k] = {"dispatches": len(fv[k]), "fetch_counter_bytes": fr,
                                 "write_counter_bytes": wr, "fetch_bytes": fr * f_fetch,
                                 "write_bytes": wr * f_write}
    return out


def main():
    p = argparse.ArgumentParser()
    p.add_argument("fetch_csv")
    p.add_argument("write_csv")
    p.add_argument("--workload", default="prefill_4k")
    a = p.parse_args()
    print(json.dumps(summarize(a.fetch_csv, a.write_csv, a.workload), indent=1))


if __name__ == "__main__":
    main()
