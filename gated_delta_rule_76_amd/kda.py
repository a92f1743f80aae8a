"""Python binding of the KDA C ABI (include/kda.h): argument marshalling only.

Every step of the layer runs in the HIP library (lib/libkda.so); this module
checks tensor shapes/dtypes/devices, allocates outputs and the workspace with
torch on the tensors' device, and passes raw pointers plus the current HIP
stream.  There is no fallback: if the library is missing or the tensors are
not on a GPU, the call raises.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

import torch

# KDA_LIBRARY may name another build of the same sources (the ABI tests use
# the host-sanitized build, lib/libkda_hostsan.so).
_LIB_PATH = os.environ.get("KDA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "lib", "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARGUMENT = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_WORKSPACE_TOO_SMALL = 3
KDA_ERR_LAUNCH = 4
KDA_F32 = 0
KDA_BF16 = 1
KDA_GATE_CHANNEL = 0
KDA_GATE_HEAD = 1
KDA_INPUT_FINAL = 0
KDA_INPUT_PREACT = 1
ABI_VERSION = 5
NOALLOC_WORKSPACE_BYTES = 128 << 20   # KDA_NOALLOC_WORKSPACE_BYTES
CHUNK = 64

_DTYPES = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}


class KdaError(RuntimeError):
    """A KDA library call returned a non-OK status."""

    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class KdaShape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("num_heads", ctypes.c_int32),
        ("d_k", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32),
        ("gate", ctypes.c_int32),
        ("input_form", ctypes.c_int32),
    ]


_lib = None


def library_path():
    return _LIB_PATH


def lib():
    """Load (once) and return the ctypes handle of libkda.so."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"KDA library not built ({_LIB_PATH} missing); "
                           "run `python -m gated_delta_rule_76_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    shp = ctypes.POINTER(KdaShape)
    L.kda_abi_version.restype = ctypes.c_int
    L.kda_abi_version.argtypes = []
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_status_string.argtypes = [ctypes.c_int]
    L.kda_prefill_workspace_size.restype = ctypes.c_int
    L.kda_prefill_workspace_size.argtypes = [shp, ctypes.POINTER(sz)]
    L.kda_prefill.restype = ctypes.c_int
    L.kda_prefill.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.kda_prefill_chunk_local.restype = ctypes.c_int
    L.kda_prefill_chunk_local.argtypes = [shp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.kda_prefill_noalloc.restype = ctypes.c_int
    L.kda_prefill_noalloc.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kda_prefill_state_pass.restype = ctypes.c_int
    L.kda_prefill_state_pass.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.kda_decode_step.restype = ctypes.c_int
    L.kda_decode_step.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kda_decode_tokens.restype = ctypes.c_int
    L.kda_decode_tokens.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kda_state_commit.restype = ctypes.c_int
    L.kda_state_commit.argtypes = [shp, vp, vp, vp, vp]
    L.kda_verify_tokens.restype = ctypes.c_int
    L.kda_verify_tokens.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kda_accept_tokens.restype = ctypes.c_int
    L.kda_accept_tokens.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kda_accept_verify_tokens.restype = ctypes.c_int
    L.kda_accept_verify_tokens.argtypes = [shp] + [vp] * 14
    L.kda_backward_workspace_size.restype = ctypes.c_int
    L.kda_backward_workspace_size.argtypes = [shp, ctypes.POINTER(sz)]
    L.kda_backward.restype = ctypes.c_int
    L.kda_backward.argtypes = [shp] + [vp] * 16 + [sz, vp]
    if L.kda_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{_LIB_PATH} has ABI version {L.kda_abi_version()}, this binding "
                           f"needs {ABI_VERSION}; rebuild with `python -m gated_delta_rule_76_amd.build`")
    _lib = L
    return L


def status_string(status):
    return lib().kda_status_string(int(status)).decode()


def _check(status, where):
    if status != KDA_OK:
        raise KdaError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_gpu(name, t, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device}); the KDA library has no CPU path")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _require_shape(name, t, shape):
    """Outputs the caller supplies must have exactly the shape the call
    writes: a smaller buffer would be written past its end on the device."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _same_device(dev, **tensors):
    """Every tensor of one call must be on one GPU: the kernels run on that
    GPU's stream and would follow the other pointers into another GPU's
    memory."""
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev} (every tensor of a call on one GPU)")


def _on(dev):
    """The call's GPU as the current device while the library runs (the
    no-allocation entry point takes its static workspace on the current
    device)."""
    return torch.cuda.device(dev) if dev.type == "cuda" else contextlib.nullcontext()


def make_shape(num_seqs, seq_len, total_tokens, num_heads, d, dtype, gate=KDA_GATE_CHANNEL,
               input_form=KDA_INPUT_FINAL):
    return KdaShape(int(num_seqs), int(seq_len), int(total_tokens), int(num_heads), int(d), int(d),
                    _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype), int(gate),
                    int(input_form))


def _gate_of(alpha, q):
    """KDA_GATE_CHANNEL when alpha has q's shape, KDA_GATE_HEAD when it has
    q's shape without the channel axis (one rate per token and head)."""
    if tuple(alpha.shape) == tuple(q.shape):
        return KDA_GATE_CHANNEL
    if tuple(alpha.shape) == tuple(q.shape[:-1]):
        return KDA_GATE_HEAD
    raise ValueError(f"alpha has shape {tuple(alpha.shape)}, expected {tuple(q.shape)} (a rate per "
                     f"key channel) or {tuple(q.shape[:-1])} (a rate per head)")


def prefill_workspace_size(num_seqs, total_tokens, num_heads, d, dtype=torch.bfloat16):
    """Recommended workspace bytes for kda_prefill (depends on N, T, H, d
    only): every chunk in one stripe.  Less works too, in stripes, down to
    the chunk table plus one record per head (plus the carried states when
    there is no final-state output)."""
    shape = make_shape(num_seqs, 0, total_tokens, num_heads, d, dtype)
    out = ctypes.c_size_t(0)
    _check(lib().kda_prefill_workspace_size(ctypes.byref(shape), ctypes.byref(out)),
           "kda_prefill_workspace_size")
    return int(out.value)


def record_bytes(d, dtype=torch.bfloat16):
    """Bytes of one chunk record (the workspace unit: one per 64-token chunk
    and head)."""
    # one sequence of 64 tokens, one head: the 256-byte chunk table + 2 records
    return (prefill_workspace_size(1, 64, 1, d, dtype) - 256) // 2


class PrefillCall:
    """A validated prefill problem: tensors, outputs and workspace bound to
    the C entry points.  ``run()`` is kda_prefill; ``chunk_local()`` and
    ``state_pass()`` are its two phases (run in that order; they need the
    recommended workspace).  Without ``workspace`` the recommended size is
    allocated, or ``workspace_bytes`` when given (the prefill then runs in
    stripes if that is less)."""

    def __init__(self, q, k, v, alpha, beta, initial_state=None, cu_seqlens=None, *,
                 output_final_state=True, workspace=None, out=None, final_state=None, preact=False,
                 allocate_workspace=True, workspace_bytes=None):
        for name, t in (("q", q), ("k", k), ("v", v)):
            _require_gpu(name, t)
        if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
            raise ValueError("q, k, v must share one dtype, float32 or bfloat16")
        _require_gpu("alpha", alpha, torch.float32)
        _require_gpu("beta", beta, torch.float32)
        dev = q.device
        if q.dim() == 4:
            if cu_seqlens is not None:
                raise ValueError("cu_seqlens needs the packed [T, H, D] layout")
            B, T, H, D = q.shape
            N, seq_len, total = B, T, B * T
        elif q.dim() == 3:
            T, H, D = q.shape
            total = T
            if cu_seqlens is None:
                N, seq_len = 1, T
            else:
                _require_gpu("cu_seqlens", cu_seqlens, torch.int32)
                if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
                    raise ValueError("cu_seqlens must be a 1-D int32 tensor [N+1]")
                N, seq_len = cu_seqlens.numel() - 1, 0
        else:
            raise ValueError("q must be [T, H, D] or [B, T, H, D]")
        gate = _gate_of(alpha, q)
        for name, t, shp in (("k", k, q.shape), ("v", v, q.shape), ("beta", beta, q.shape[:-1])):
            if tuple(t.shape) != tuple(shp):
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shp)}")
        if initial_state is not None:
            _require_gpu("initial_state", initial_state, torch.float32)
            if tuple(initial_state.shape) != (N, H, D, D):
                raise ValueError(f"initial_state must be {(N, H, D, D)}")
        self.shape = make_shape(N, seq_len, total, H, D, q.dtype, gate,
                                KDA_INPUT_PREACT if preact else KDA_INPUT_FINAL)
        self.o = out if out is not None else torch.empty(v.shape, dtype=torch.float32, device=dev)
        _require_gpu("out", self.o, torch.float32)
        _require_shape("out", self.o, v.shape)
        self.S_T = None
        if output_final_state:
            self.S_T = (final_state if final_state is not None
                        else torch.empty((N, H, D, D), dtype=torch.float32, device=dev))
            _require_gpu("final_state", self.S_T, torch.float32)
            _require_shape("final_state", self.S_T, (N, H, D, D))
        _same_device(dev, k=k, v=v, alpha=alpha, beta=beta, cu_seqlens=cu_seqlens, initial_state=initial_state,
                     out=self.o, final_state=self.S_T)
        if workspace is None and allocate_workspace:
            need = (workspace_bytes if workspace_bytes is not None
                    else prefill_workspace_size(N, total, H, D, q.dtype))
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        if workspace is not None:
            _require_gpu("workspace", workspace)
        _same_device(dev, workspace=workspace)
        self.workspace = workspace
        self.device = dev
        self._t = (q, k, v, alpha, beta, cu_seqlens, initial_state)

    def _ws(self):
        if self.workspace is None:
            return None, 0
        return _ptr(self.workspace), self.workspace.numel() * self.workspace.element_size()

    def run(self):
        q, k, v, alpha, beta, cu, S0 = self._t
        ws, nb = self._ws()
        with _on(self.device):
            _check(lib().kda_prefill(ctypes.byref(self.shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                     _ptr(beta), _ptr(cu), _ptr(S0), _ptr(self.o), _ptr(self.S_T), ws, nb,
                                     _stream(self.device)), "kda_prefill")
        return self.o, self.S_T

    def run_noalloc(self):
        """kda_prefill_noalloc: the same call with the library's static
        workspace (no workspace tensor is used or needed)."""
        q, k, v, alpha, beta, cu, S0 = self._t
        with _on(self.device):
            _check(lib().kda_prefill_noalloc(ctypes.byref(self.shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                             _ptr(beta), _ptr(cu), _ptr(S0), _ptr(self.o), _ptr(self.S_T),
                                             _stream(self.device)), "kda_prefill_noalloc")
        return self.o, self.S_T

    def chunk_local(self):
        q, k, _, alpha, beta, cu, _ = self._t
        ws, nb = self._ws()
        with _on(self.device):
            _check(lib().kda_prefill_chunk_local(ctypes.byref(self.shape), _ptr(q), _ptr(k), _ptr(alpha),
                                                 _ptr(beta), _ptr(cu), ws, nb, _stream(self.device)),
                   "kda_prefill_chunk_local")

    def state_pass(self):
        q, k, v, alpha, _, cu, S0 = self._t
        ws, nb = self._ws()
        with _on(self.device):
            _check(lib().kda_prefill_state_pass(ctypes.byref(self.shape), _ptr(q), _ptr(k), _ptr(v),
                                                _ptr(alpha), _ptr(cu), _ptr(S0), _ptr(self.o),
                                                _ptr(self.S_T), ws, nb, _stream(self.device)),
                   "kda_prefill_state_pass")
        return self.o, self.S_T


def prefill(q, k, v, alpha, beta, initial_state=None, cu_seqlens=None, *,
            output_final_state=True, workspace=None, out=None, final_state=None, preact=False,
            workspace_bytes=None):
    """Chunked KDA prefill.  Returns (o, S_T).

    Layouts: q, k, alpha [T, H, D] with v [T, H, D] (one sequence, or a
    packed varlen batch when ``cu_seqlens`` [N+1] int32 is given), or
    [B, T, H, D] for a dense batch of B equal-length sequences; beta
    [T, H] / [B, T, H].  q, k, v are bf16 or fp32; alpha, beta fp32.
    alpha of beta's shape (one rate per token and head) selects the
    scalar-gate form.  With ``preact=True``, q and k are raw (the library
    scales them to unit length), alpha holds decay pre-activations a
    (alpha = exp(-softplus(a))) and beta holds b (beta = sigmoid(b)).
    initial_state [N, H, D, D] fp32 or None (zeros).  o is fp32 with v's
    shape; S_T is [N, H, D, D] fp32 (None if output_final_state is False).
    ``final_state`` may be ``initial_state`` for an in-place update.
    ``workspace`` (uint8 device tensor) or ``workspace_bytes`` bound the
    scratch memory; by default the recommended size is allocated.
    """
    return PrefillCall(q, k, v, alpha, beta, initial_state, cu_seqlens,
                       output_final_state=output_final_state, workspace=workspace, out=out,
                       final_state=final_state, preact=preact, workspace_bytes=workspace_bytes).run()


def prefill_noalloc(q, k, v, alpha, beta, initial_state=None, cu_seqlens=None, *,
                    output_final_state=True, out=None, final_state=None, preact=False):
    """``prefill`` through kda_prefill_noalloc: the library's static device
    workspace instead of a workspace tensor (for callers that cannot allocate
    device memory; longer batches run in stripes, and batches whose minimum
    workspace exceeds NOALLOC_WORKSPACE_BYTES are rejected).  Outputs are allocated here unless ``out`` / ``final_state``
    are given."""
    return PrefillCall(q, k, v, alpha, beta, initial_state, cu_seqlens,
                       output_final_state=output_final_state, out=out, final_state=final_state,
                       preact=preact, allocate_workspace=False).run_noalloc()


def decode_step(q, k, v, alpha, beta, state, out=None, preact=False):
    """One decode step for N sequences: q, k, v, alpha [N, H, D]; beta [N, H];
    state [N, H, D, D] fp32 updated in place.  Returns o [N, H, D] fp32.
    alpha [N, H] (one rate per head) selects the scalar-gate form;
    ``preact=True`` as for ``prefill``."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require_gpu(name, t)
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, float32 or bfloat16")
    _require_gpu("alpha", alpha, torch.float32)
    _require_gpu("beta", beta, torch.float32)
    _require_gpu("state", state, torch.float32)
    if q.dim() != 3:
        raise ValueError("decode inputs are [N, H, D]")
    N, H, D = q.shape
    gate = _gate_of(alpha, q)
    for name, t, shp in (("k", k, q.shape), ("v", v, q.shape),
                         ("beta", beta, q.shape[:-1]), ("state", state, (N, H, D, D))):
        if tuple(t.shape) != tuple(shp):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shp)}")
    o = out if out is not None else torch.empty((N, H, D), dtype=torch.float32, device=q.device)
    _require_gpu("out", o, torch.float32)
    _require_shape("out", o, (N, H, D))
    _same_device(q.device, k=k, v=v, alpha=alpha, beta=beta, state=state, out=o)
    shape = make_shape(N, 1, N, H, D, q.dtype, gate, KDA_INPUT_PREACT if preact else KDA_INPUT_FINAL)
    with _on(q.device):
        st = lib().kda_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                   _ptr(state), _ptr(o), _stream(q.device))
    _check(st, "kda_decode_step")
    return o


def decode_tokens(q, k, v, alpha, beta, state, keep_states=False, preact=False, out=None,
                  states=None):
    """k new tokens for each of N sequences from the live states.

    q, k, v [N, k, H, D]; alpha [N, k, H, D] (or [N, k, H]: scalar gate);
    beta [N, k, H]; state [N, H, D, D] fp32.  Returns o [N, k, H, D] fp32.
    keep_states=False advances ``state`` in place by all k tokens.
    keep_states=True leaves ``state`` as it is and also returns the state
    after every token, [N, k, H, D, D] fp32 (``states`` may be given), for
    ``state_commit``: returns (o, states).
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require_gpu(name, t)
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, float32 or bfloat16")
    _require_gpu("alpha", alpha, torch.float32)
    _require_gpu("beta", beta, torch.float32)
    _require_gpu("state", state, torch.float32)
    if q.dim() != 4:
        raise ValueError("multi-token decode inputs are [N, k, H, D]")
    N, K, H, D = q.shape
    gate = _gate_of(alpha, q)
    for name, t, shp in (("k", k, q.shape), ("v", v, q.shape), ("beta", beta, q.shape[:-1]),
                         ("state", state, (N, H, D, D))):
        if tuple(t.shape) != tuple(shp):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shp)}")
    o = out if out is not None else torch.empty((N, K, H, D), dtype=torch.float32, device=q.device)
    _require_gpu("out", o, torch.float32)
    _require_shape("out", o, (N, K, H, D))
    hist = None
    if keep_states:
        hist = states if states is not None else torch.empty((N, K, H, D, D), dtype=torch.float32,
                                                             device=q.device)
        _require_gpu("states", hist, torch.float32)
        if tuple(hist.shape) != (N, K, H, D, D):
            raise ValueError(f"states must be {(N, K, H, D, D)}")
    _same_device(q.device, k=k, v=v, alpha=alpha, beta=beta, state=state, out=o, states=hist)
    shape = make_shape(N, K, N * K, H, D, q.dtype, gate, KDA_INPUT_PREACT if preact else KDA_INPUT_FINAL)
    with _on(q.device):
        _check(lib().kda_decode_tokens(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                       _ptr(beta), _ptr(state), _ptr(o), _ptr(hist), _stream(q.device)),
               "kda_decode_tokens")
    return (o, hist) if keep_states else o


def _token_round(q, k, v, alpha, beta, state, preact):
    """Checks shared by verify_tokens and accept_tokens; returns (N, K, H, D,
    shape struct)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require_gpu(name, t)
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, float32 or bfloat16")
    _require_gpu("alpha", alpha, torch.float32)
    _require_gpu("beta", beta, torch.float32)
    _require_gpu("state", state, torch.float32)
    if q.dim() != 4:
        raise ValueError("multi-token decode inputs are [N, k, H, D]")
    N, K, H, D = q.shape
    gate = _gate_of(alpha, q)
    for name, t, shp in (("k", k, q.shape), ("v", v, q.shape), ("beta", beta, q.shape[:-1]),
                         ("state", state, (N, H, D, D))):
        if tuple(t.shape) != tuple(shp):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shp)}")
    shape = make_shape(N, K, N * K, H, D, q.dtype, gate, KDA_INPUT_PREACT if preact else KDA_INPUT_FINAL)
    return N, K, H, D, shape


def verify_tokens(q, k, v, alpha, beta, state, preact=False, out=None):
    """Outputs of k drafted tokens per sequence from the live states, which
    are left as they are (verification with rollback by recomputation: pair
    with ``accept_tokens``).  Inputs as for ``decode_tokens``; returns o
    [N, k, H, D] fp32."""
    N, K, H, D, shape = _token_round(q, k, v, alpha, beta, state, preact)
    o = out if out is not None else torch.empty((N, K, H, D), dtype=torch.float32, device=q.device)
    _require_gpu("out", o, torch.float32)
    _require_shape("out", o, (N, K, H, D))
    _same_device(q.device, k=k, v=v, alpha=alpha, beta=beta, state=state, out=o)
    with _on(q.device):
        _check(lib().kda_verify_tokens(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                       _ptr(beta), _ptr(state), _ptr(o), _stream(q.device)),
               "kda_verify_tokens")
    return o


def accept_tokens(q, k, v, alpha, beta, state, accepted, preact=False):
    """Advance state[n] in place by the first accepted[n] of the k tokens
    (clamped to [0, k]) that ``verify_tokens`` checked; accepted: int32 [N]
    on the GPU.  Returns ``state``."""
    N, K, H, D, shape = _token_round(q, k, v, alpha, beta, state, preact)
    _require_gpu("accepted", accepted, torch.int32)
    if tuple(accepted.shape) != (N,):
        raise ValueError(f"accepted has shape {tuple(accepted.shape)}, expected {(N,)}")
    _same_device(q.device, k=k, v=v, alpha=alpha, beta=beta, state=state, accepted=accepted)
    with _on(q.device):
        _check(lib().kda_accept_tokens(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                       _ptr(beta), _ptr(state), _ptr(accepted), _stream(q.device)),
               "kda_accept_tokens")
    return state


def accept_verify_tokens(prev, accepted, q, k, v, alpha, beta, state, preact=False, out=None):
    """One verification round in one pass over the state: ``state`` advanced
    in place by the first accepted[n] tokens of the previous round, ``prev`` =
    (q, k, v, alpha, beta) of that round, then the outputs of this round's
    tokens from it (equal to accept_tokens(*prev, state, accepted) then
    verify_tokens(q, k, v, alpha, beta, state)).  Returns o [N, k, H, D]."""
    return AcceptVerifyCall(prev, accepted, q, k, v, alpha, beta, state, preact=preact, out=out).run()


class AcceptVerifyCall:
    """A validated ``accept_verify_tokens`` round bound to its tensors, for
    loops that issue it many times: the checks and the pointer marshalling run
    once, ``run()`` makes only the C call (on the current stream of the
    tensors' device)."""

    def __init__(self, prev, accepted, q, k, v, alpha, beta, state, preact=False, out=None):
        q0, k0, v0, alpha0, beta0 = prev
        N, K, H, D, shape = _token_round(q, k, v, alpha, beta, state, preact)
        N0, K0, H0, D0, shape0 = _token_round(q0, k0, v0, alpha0, beta0, state, preact)
        if (N0, K0, H0, D0) != (N, K, H, D) or q0.dtype != q.dtype or shape0.gate != shape.gate:
            raise ValueError("the previous round's tokens must have this round's shape, dtype and gate kind")
        _require_gpu("accepted", accepted, torch.int32)
        if tuple(accepted.shape) != (N,):
            raise ValueError(f"accepted has shape {tuple(accepted.shape)}, expected {(N,)}")
        self.o = out if out is not None else torch.empty((N, K, H, D), dtype=torch.float32, device=q.device)
        _require_gpu("out", self.o, torch.float32)
        _require_shape("out", self.o, (N, K, H, D))
        _same_device(q.device, k=k, v=v, alpha=alpha, beta=beta, state=state, out=self.o, q0=q0, k0=k0, v0=v0,
                     alpha0=alpha0, beta0=beta0, accepted=accepted)
        self.shape = shape
        self.device = q.device
        self._keep = (q0, k0, v0, alpha0, beta0, accepted, q, k, v, alpha, beta, state)  # keep them alive
        self._args = [_ptr(t) for t in self._keep] + [_ptr(self.o)]

    def run(self):
        with _on(self.device):
            _check(lib().kda_accept_verify_tokens(ctypes.byref(self.shape), *self._args, _stream(self.device)),
                   "kda_accept_verify_tokens")
        return self.o


def state_commit(state, states, accepted):
    """state[n] <- states[n, accepted[n] - 1] for accepted[n] >= 1 (capped at
    k); accepted[n] <= 0 keeps state[n].  accepted: int32 [N] on the GPU."""
    _require_gpu("state", state, torch.float32)
    _require_gpu("states", states, torch.float32)
    _require_gpu("accepted", accepted, torch.int32)
    if states.dim() != 5 or state.dim() != 4:
        raise ValueError("state is [N, H, D, D] and states [N, k, H, D, D]")
    N, K, H, D, _ = states.shape
    if tuple(state.shape) != (N, H, D, D) or tuple(accepted.shape) != (N,):
        raise ValueError("state, states and accepted disagree in shape")
    _same_device(state.device, states=states, accepted=accepted)
    shape = make_shape(N, K, N * K, H, D, torch.float32)
    with _on(state.device):
        _check(lib().kda_state_commit(ctypes.byref(shape), _ptr(state), _ptr(states), _ptr(accepted),
                                      _stream(state.device)), "kda_state_commit")
    return state


def backward_workspace_size(num_seqs, total_tokens, num_heads, d, dtype=torch.bfloat16, gate=KDA_GATE_CHANNEL):
    shape = make_shape(num_seqs, 0, total_tokens, num_heads, d, dtype, gate)
    out = ctypes.c_size_t(0)
    _check(lib().kda_backward_workspace_size(ctypes.byref(shape), ctypes.byref(out)),
           "kda_backward_workspace_size")
    return int(out.value)


def backward(q, k, v, alpha, beta, dO, initial_state=None, dS_T=None, cu_seqlens=None, *,
             want_dS0=True, workspace=None, workspace_bytes=None):
    """Gradients of the layer: returns (dq, dk, dv, dalpha, dbeta, dS0), all
    fp32 (dS0 None if want_dS0 is False).  Inputs as for ``prefill`` (packed
    [T, H, D] with optional cu_seqlens, or [B, T, H, D]); dO has v's shape
    (fp32), dS_T the final states' shape (fp32) or None for zero.
    ``workspace`` (uint8 device tensor) or ``workspace_bytes`` bound the
    scratch memory (below the recommended size the sequences run in pieces);
    by default the recommended size is allocated."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require_gpu(name, t)
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, float32 or bfloat16")
    _require_gpu("alpha", alpha, torch.float32)
    _require_gpu("beta", beta, torch.float32)
    _require_gpu("dO", dO, torch.float32)
    dev = q.device
    if q.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs the packed [T, H, D] layout")
        B, T, H, D = q.shape
        N, seq_len, total = B, T, B * T
    elif q.dim() == 3:
        T, H, D = q.shape
        total = T
        if cu_seqlens is None:
            N, seq_len = 1, T
        else:
            _require_gpu("cu_seqlens", cu_seqlens, torch.int32)
            N, seq_len = cu_seqlens.numel() - 1, 0
    else:
        raise ValueError("q must be [T, H, D] or [B, T, H, D]")
    gate = _gate_of(alpha, q)
    for name, t, shp in (("k", k, q.shape), ("v", v, q.shape), ("beta", beta, q.shape[:-1]),
                         ("dO", dO, v.shape)):
        if tuple(t.shape) != tuple(shp):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shp)}")
    for name, t in (("initial_state", initial_state), ("dS_T", dS_T)):
        if t is not None:
            _require_gpu(name, t, torch.float32)
            if tuple(t.shape) != (N, H, D, D):
                raise ValueError(f"{name} must be {(N, H, D, D)}")
    shape = make_shape(N, seq_len, total, H, D, q.dtype, gate)
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty(q.shape, **f32), torch.empty(k.shape, **f32), torch.empty(v.shape, **f32)
    dalpha, dbeta = torch.empty(alpha.shape, **f32), torch.empty(beta.shape, **f32)
    dS0 = torch.empty((N, H, D, D), **f32) if want_dS0 else None
    need = ctypes.c_size_t(0)
    _check(lib().kda_backward_workspace_size(ctypes.byref(shape), ctypes.byref(need)),
           "kda_backward_workspace_size")
    if workspace is None:
        nbytes = int(need.value) if workspace_bytes is None else int(workspace_bytes)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _require_gpu("workspace", workspace)
    _same_device(dev, k=k, v=v, alpha=alpha, beta=beta, dO=dO, cu_seqlens=cu_seqlens,
                 initial_state=initial_state, dS_T=dS_T, workspace=workspace)
    with _on(dev):
        _check(lib().kda_backward(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                  _ptr(cu_seqlens), _ptr(initial_state), _ptr(dO), _ptr(dS_T), _ptr(dq),
                                  _ptr(dk), _ptr(dv), _ptr(dalpha), _ptr(dbeta), _ptr(dS0), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(dev)),
               "kda_backward")
    return dq, dk, dv, dalpha, dbeta, dS0
