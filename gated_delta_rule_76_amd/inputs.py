"""Seeded synthetic inputs for the KDA layer (no KDA arithmetic in here).

This module is shared by the tests, the benchmark and the smoke check: it
draws the random tensors that both the HIP library and the CPU oracle
consume.  It holds none of the layer's own arithmetic -- only random draws,
the input distributions (L2-normalised q and k, sigmoid beta,
exp(-softplus(.)) decay) and packing.  It imports nothing from the library
binding, so it can be used on a machine without a GPU.

Distributions (per the workloads the layer is measured on):
  q, k     N(0,1) per element, then L2-normalised over the head dimension
           per (token, head), in fp32, then cast to the q/k/v dtype;
  v        N(0,1), cast to the q/k/v dtype;
  beta     sigmoid(N(0,1)) per (token, head), fp32;
  alpha    exp(-softplus(N(0,1) + shift)) per (token, head, key channel),
           fp32; shift 0 ("medium", mean ~0.5), +2 ("strong", mean
           ~0.14, the prefill/decode workloads), -4 ("weak", mean ~0.97);
           with gate="head" the same law with one draw per (token, head)
           (the scalar-gate form);
  form     "final" gives the tensors above; "preact" gives what they are
           made from: raw q, k (N(0,1), not normalised, cast to the q/k/v
           dtype), a = N(0,1) + shift in alpha's place and b = N(0,1) in
           beta's (the same draws);
  state    std * N(0,1) fp32 (std 0.02 for the varlen and decode workloads);
  lengths  uniform integers in [lo, hi] inclusive.

Draw order and seeding: every tensor has its own stream id and is drawn in
blocks of 65,536 tokens (bounding the temporaries of very long inputs),
block b of stream s seeded with seed * 1_000_003 + 7919 * s + b.  Lengths use a CPU generator; everything
else uses a generator on ``device`` (CPU and GPU generators give different
numbers, which is fine: the oracle always consumes the exact tensors the GPU
consumed, copied back).
"""

from __future__ import annotations

import torch

DECAY_SHIFT = {"medium": 0.0, "strong": 2.0, "weak": -4.0}
BLOCK_TOKENS = 65536

_STREAM = {"q": 1, "k": 2, "v": 3, "alpha": 4, "beta": 5, "state": 6, "lengths": 7, "dO": 8,
           "dS_T": 9}


def _generator(device, seed, stream, block):
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + 7919 * stream + block) % (2**62))
    return g


def _randn_tokens(shape, seed, stream, device):
    """N(0,1) fp32 of ``shape`` whose first axis is tokens, drawn blockwise."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    T = shape[0]
    for b, t0 in enumerate(range(0, T, BLOCK_TOKENS)):
        t1 = min(T, t0 + BLOCK_TOKENS)
        g = _generator(device, seed, stream, b)
        out[t0:t1] = torch.randn((t1 - t0,) + tuple(shape[1:]), generator=g, device=device)
    return out


def _unit(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)


def varlen_lengths(n, lo, hi, seed=0):
    """n sequence lengths, uniform integers in [lo, hi] inclusive (CPU draw)."""
    g = _generator("cpu", seed, _STREAM["lengths"], 0)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def token_inputs(T, H, D, dtype=torch.bfloat16, decay="strong", seed=0, device="cpu", dv=None,
                 gate="channel", form="final"):
    """q, k, v, alpha, beta for T tokens x H heads (token-major layout).

    Returns a dict: q, k [T,H,D] and v [T,H,dv] in ``dtype``; alpha [T,H,D]
    (gate="channel") or [T,H] (gate="head") and beta [T,H] fp32.
    """
    if gate not in ("channel", "head"):
        raise ValueError("gate is 'channel' or 'head'")
    if form not in ("final", "preact"):
        raise ValueError("form is 'final' or 'preact'")
    pre = form == "preact"
    dv = D if dv is None else dv
    shift = DECAY_SHIFT[decay]
    unit = (lambda x: x) if pre else _unit
    q = unit(_randn_tokens((T, H, D), seed, _STREAM["q"], device)).to(dtype)
    k = unit(_randn_tokens((T, H, D), seed, _STREAM["k"], device)).to(dtype)
    v = _randn_tokens((T, H, dv), seed, _STREAM["v"], device).to(dtype)
    a = _randn_tokens((T, H, D) if gate == "channel" else (T, H), seed, _STREAM["alpha"], device)
    alpha = a + shift if pre else torch.exp(-torch.nn.functional.softplus(a + shift))
    del a
    b = _randn_tokens((T, H), seed, _STREAM["beta"], device)
    beta = b if pre else torch.sigmoid(b)
    return {"q": q, "k": k, "v": v, "alpha": alpha.contiguous(), "beta": beta.contiguous()}


def state(N, H, D, std=0.02, seed=0, device="cpu", dv=None, stream_offset=0):
    """std * N(0,1) fp32 state [N, H, D, dv]."""
    dv = D if dv is None else dv
    g = _generator(device, seed, _STREAM["state"] + 16 * stream_offset, 0)
    return (std * torch.randn((N, H, D, dv), generator=g, device=device)).contiguous()


def prefill_inputs(lengths, H, D, dtype=torch.bfloat16, decay="strong", s0_std=None,
                   seed=0, device="cpu", gate="channel", form="final"):
    """Packed prefill batch for sequences of the given lengths.

    Returns token_inputs(...) plus ``cu_seqlens`` (int32 [N+1], on device),
    ``lengths`` (list) and ``S0`` (fp32 [N,H,D,D], or None when s0_std is
    None, meaning a zero initial state).
    """
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    d = token_inputs(T, H, D, dtype, decay, seed, device, gate=gate, form=form)
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=device)
    d["lengths"] = lengths
    d["S0"] = None if s0_std is None else state(len(lengths), H, D, s0_std, seed, device)
    return d


def decode_inputs(B, H, D, steps, dtype=torch.bfloat16, decay="strong", s_std=0.02,
                  seed=0, device="cpu", gate="channel", form="final"):
    """State [B,H,D,D] plus ``steps`` per-step token sets stacked on axis 0.

    Returns dict: S fp32 [B,H,D,D]; q, k, v [steps,B,H,D]; alpha [steps,B,H,D]
    (or [steps,B,H] with gate="head"); beta [steps,B,H].  Step s uses token row s*B .. s*B+B-1 of one draw of
    steps*B tokens.
    """
    t = token_inputs(steps * B, H, D, dtype, decay, seed, device, gate=gate, form=form)
    out = {name: x.reshape((steps, B) + tuple(x.shape[1:])) for name, x in t.items()}
    out["S"] = state(B, H, D, s_std, seed, device)
    return out


def grad_inputs(T, H, D, N, seed=0, device="cpu", dS_std=0.02):
    """Upstream gradients for the backward pass: dL/do ~ N(0,1) fp32
    [T, H, D] and dL/dS_T ~ dS_std * N(0,1) fp32 [N, H, D, D] (None when
    dS_std is None)."""
    dO = _randn_tokens((T, H, D), seed, _STREAM["dO"], device)
    dST = None
    if dS_std is not None:
        g = _generator(device, seed, _STREAM["dS_T"], 0)
        dST = (dS_std * torch.randn((N, H, D, D), generator=g, device=device)).contiguous()
    return dO, dST


# The measured workloads, named by what they are.
WORKLOADS = {
    "tiny_fp32": dict(kind="prefill", lengths=[64], H=2, D=16, dtype="float32",
                      decay="medium", s0_std=None),
    "prefill_4k": dict(kind="prefill", lengths=[4096], H=32, D=128, dtype="bfloat16",
                       decay="strong", s0_std=None),
    "varlen_8seq": dict(kind="prefill", lengths=("uniform", 8, 1024, 16384), H=32, D=128,
                        dtype="bfloat16", decay="strong", s0_std=0.02),
    "decode_b256": dict(kind="decode", B=256, H=32, D=128, steps=100, dtype="bfloat16",
                        decay="strong", s_std=0.02),
    "long_1m": dict(kind="prefill", lengths=[1 << 20], H=32, D=128, dtype="bfloat16",
                    decay="strong", s0_std=None),
}


def workload_lengths(spec, seed=0):
    L = spec["lengths"]
    if isinstance(L, tuple) and L[0] == "uniform":
        return varlen_lengths(L[1], L[2], L[3], seed)
    return list(L)
