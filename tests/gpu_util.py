"""Helpers for the GPU parity tests (device selection, copies to fp64 numpy)."""

import numpy as np
import pytest
import torch


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def seeded_sample(n_total, n_pick, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n_total, size=min(n_pick, n_total), replace=False))


def parity(o, ST, ro, rST, tol, what, cu_seqlens=None):
    """Element-by-element comparison of a prefill result with the oracle.

    o [T, H, d_v] and S_T [N, H, d_k, d_v] (GPU tensors or arrays) against
    ro, rST (float64).  Asserts rel-L2 <= tol over each whole tensor and over
    every (sequence, head) slice of o and of S_T, and reports the worst
    (sequence, head) and the largest absolute error in the failure message.
    Returns the summary dict."""
    o = np64(o) if hasattr(o, "detach") else np.asarray(o, dtype=np.float64)
    ST = np64(ST) if hasattr(ST, "detach") else np.asarray(ST, dtype=np.float64)
    T, H = ro.shape[:2]
    N = rST.shape[0]
    cu = (np.asarray(cu_seqlens, dtype=np.int64) if cu_seqlens is not None
          else np.arange(N + 1, dtype=np.int64) * (T // max(N, 1)))

    def rel(x, r):
        den = np.linalg.norm(r)
        num = np.linalg.norm(x - r)
        return 0.0 if num == 0.0 else (float("inf") if den == 0.0 else float(num / den))

    worst_o, worst_s = (0.0, None), (0.0, None)
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            if e > s:
                r = rel(o[s:e, h], ro[s:e, h])
                if r >= worst_o[0]:
                    worst_o = (r, (n, h))
            r = rel(ST[n, h], rST[n, h])
            if r >= worst_s[0]:
                worst_s = (r, (n, h))
    rep = {"o": rel(o, ro), "S_T": rel(ST, rST), "worst_o": worst_o, "worst_S_T": worst_s,
           "maxabs_o": float(np.max(np.abs(o - ro))) if o.size else 0.0,
           "maxabs_S_T": float(np.max(np.abs(ST - rST))) if ST.size else 0.0}
    msg = (f"{what}: rel-L2 o {rep['o']:.3e} S_T {rep['S_T']:.3e}; worst (seq, head) o "
           f"{worst_o[0]:.3e} at {worst_o[1]}, S_T {worst_s[0]:.3e} at {worst_s[1]}; max |err| o "
           f"{rep['maxabs_o']:.3e} S_T {rep['maxabs_S_T']:.3e} (tol {tol})")
    assert rep["o"] <= tol and rep["S_T"] <= tol and worst_o[0] <= tol and worst_s[0] <= tol, msg
    return rep
