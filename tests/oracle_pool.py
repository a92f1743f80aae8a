"""Run the fp64 oracle over groups of heads in child processes.

Heads are independent in the update rule, so the oracle of a [T, H, ...]
problem is the oracle of each head group, concatenated along the head axis.
Each group runs in a fresh interpreter started with subprocess (it imports
numpy and the oracle only, so it never holds a GPU context, whatever the
calling process holds); inputs go to it and results come back through pipes
in numpy's .npy format.  Inputs travel as float32 (bf16 values are exact in
float32); the oracle converts them to float64 before any arithmetic.
"""

from __future__ import annotations

import io
import os
import subprocess
import sys
import threading

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MAX_WORKERS = 16

_CHILD = r"""
import importlib, io, sys
import numpy as np
module, name = sys.argv[1], sys.argv[2]
fn = getattr(importlib.import_module(module), name)
buf = io.BytesIO(sys.stdin.buffer.read())
arrs = [np.load(buf) for _ in range(5)]
flags = np.load(buf)
S0 = np.load(buf) if flags[0] else None
cu = np.load(buf) if flags[1] else None
o, ST = fn(*arrs, S0, cu_seqlens=cu)
out = io.BytesIO()
np.save(out, o)
np.save(out, ST)
sys.stdout.buffer.write(out.getvalue())
"""


def _job_bytes(arrs, S0, cu):
    b = io.BytesIO()
    for a in arrs:
        np.save(b, a)
    np.save(b, np.array([S0 is not None, cu is not None]))
    if S0 is not None:
        np.save(b, S0)
    if cu is not None:
        np.save(b, cu)
    return b.getvalue()


def per_head(fn, q, k, v, alpha, beta, S0=None, cu_seqlens=None, workers=None, timeout=600):
    """(o, S_T) of ``fn`` (an oracle prefill function taking q, k, v, alpha,
    beta, S0 and cu_seqlens=...) over all heads, computed in head groups.

    q, k, alpha: [T, H, ...]; v: [T, H, d_v]; beta: [T, H]; S0: [N, H, d_k,
    d_v] or None (numpy arrays or CPU tensors convertible with np.asarray)."""
    arrs = [np.asarray(x, dtype=np.float32) for x in (q, k, v, alpha, beta)]
    S0 = None if S0 is None else np.asarray(S0, dtype=np.float64)
    cu = None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    H = arrs[0].shape[1]
    n = workers or max(1, min(MAX_WORKERS, os.cpu_count() or 1, H))
    groups = [g for g in np.array_split(np.arange(H), n) if len(g)]
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1",
               PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    results = [None] * len(groups)
    errors = []

    def run(i, g):
        data = _job_bytes([np.ascontiguousarray(a[:, g]) for a in arrs],
                          None if S0 is None else np.ascontiguousarray(S0[:, g]), cu)
        p = subprocess.Popen([sys.executable, "-c", _CHILD, fn.__module__, fn.__name__], cwd=ROOT,
                             env=env, stdin=subprocess.PIPE, stdout=subprocess.PIPE,
                             stderr=subprocess.PIPE)
        out, err = p.communicate(data, timeout=timeout)
        if p.returncode != 0:
            errors.append(f"oracle worker {i} failed ({p.returncode}): {err.decode()[-2000:]}")
            return
        buf = io.BytesIO(out)
        results[i] = (np.load(buf), np.load(buf))

    threads = [threading.Thread(target=run, args=(i, g)) for i, g in enumerate(groups)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    if errors:
        raise RuntimeError("\n".join(errors))
    o = np.concatenate([r[0] for r in results], axis=1)
    ST = np.concatenate([r[1] for r in results], axis=1)
    return o, ST
