"""Pins for the backward oracle, oracle/backward.py.

What fixes it other than itself:
  * torch.autograd in float64 through a forward recurrence written here with
    the printed matrices (I - beta k k^T), Diag(alpha) and beta k v^T formed
    explicitly (a library routine differentiating an independent forward);
  * central finite differences of the pinned forward oracle (kda_recurrent /
    gdn_recurrent) on tiny inputs;
  * a closed form: alpha = 1, beta = 0 keeps S_t = S0, so dq_t = S0 dO_t and
    dS0 = dS_T + sum_t q_t dO_t^T, with dk = dv = 0;
and each planted mistake below fails at least one of them.
"""

import numpy as np
import pytest
import torch

from oracle import gdn_recurrent, kda_recurrent
from oracle import backward as bw


def _case(seed, T, H, dk, dv, per_head=False, cu=None, with_s0=True, with_dst=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    alpha = rng.uniform(0.4, 1.0, (T, H) if per_head else (T, H, dk))
    beta = rng.uniform(0.1, 0.9, (T, H))
    N = 1 if cu is None else len(cu) - 1
    S0 = rng.standard_normal((N, H, dk, dv)) if with_s0 else None
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((N, H, dk, dv)) if with_dst else None
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0, dO=dO, dST=dST, cu=cu)


def _autograd(c):
    """Gradients by torch.autograd of L = sum(o * dO) + sum(S_T * dS_T)."""
    t = {n: torch.tensor(c[n], dtype=torch.float64, requires_grad=True)
         for n in ("q", "k", "v", "alpha", "beta")}
    T, H, dk = c["q"].shape
    dv = c["v"].shape[-1]
    cu = [0, T] if c["cu"] is None else list(c["cu"])
    S0 = None if c["S0"] is None else torch.tensor(c["S0"], dtype=torch.float64, requires_grad=True)
    eye = torch.eye(dk, dtype=torch.float64)
    loss = 0.0
    for n in range(len(cu) - 1):
        for h in range(H):
            S = torch.zeros(dk, dv, dtype=torch.float64) if S0 is None else S0[n, h]
            for s in range(cu[n], cu[n + 1]):
                kk = t["k"][s, h][:, None]
                a = t["alpha"][s, h]
                D = torch.diag(a.expand(dk)) if a.dim() == 0 else torch.diag(a)
                S = (eye - t["beta"][s, h] * kk @ kk.T) @ D @ S + t["beta"][s, h] * kk @ t["v"][s, h][None, :]
                loss = loss + (S.T @ t["q"][s, h] * torch.tensor(c["dO"][s, h])).sum()
            if c["dST"] is not None:
                loss = loss + (S * torch.tensor(c["dST"][n, h])).sum()
    loss.backward()
    g = {n: t[n].grad.numpy() for n in t}
    g["S0"] = None if S0 is None else S0.grad.numpy()
    return g


def _oracle(c, fn=bw.kda_backward):
    return fn(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["dO"], c["S0"], c["dST"], c["cu"])


def pin_autograd(fn):
    ok = True
    for c in (_case(1, 9, 2, 4, 3), _case(2, 12, 2, 3, 3, per_head=True, cu=[0, 5, 5, 12]),
              _case(3, 7, 1, 4, 4, with_s0=False, with_dst=False)):
        dq, dk, dv, da, db, dS0 = _oracle(c, fn)
        g = _autograd(c)
        for got, want in ((dq, g["q"]), (dk, g["k"]), (dv, g["v"]), (da, g["alpha"]), (db, g["beta"])):
            ok = ok and np.allclose(got, want, rtol=1e-10, atol=1e-10)
        if g["S0"] is not None:
            ok = ok and np.allclose(dS0, g["S0"], rtol=1e-10, atol=1e-10)
    return ok


def _loss(c, **override):
    x = dict(c, **override)
    run = gdn_recurrent if x["alpha"].ndim == 2 else kda_recurrent
    o, ST = run(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], cu_seqlens=x["cu"])
    return np.sum(o * x["dO"]) + (0.0 if x["dST"] is None else np.sum(ST * x["dST"]))


def pin_finite_differences(fn):
    ok = True
    for c in (_case(4, 6, 1, 3, 2), _case(5, 5, 2, 3, 3, per_head=True)):
        grads = dict(zip(("q", "k", "v", "alpha", "beta", "S0"), _oracle(c, fn)))
        rng = np.random.default_rng(6)
        for name in ("q", "k", "v", "alpha", "beta", "S0"):
            x = c[name]
            for _ in range(4):
                idx = tuple(int(rng.integers(0, s)) for s in x.shape)
                e = np.zeros_like(x)
                e[idx] = 1e-6
                fd = (_loss(c, **{name: x + e}) - _loss(c, **{name: x - e})) / 2e-6
                ok = ok and abs(fd - grads[name][idx]) <= 1e-7 * max(1.0, abs(fd))
    return ok


def pin_identity_closed_form(fn):
    c = _case(7, 8, 2, 4, 3)
    c["alpha"] = np.ones_like(c["alpha"])
    c["beta"] = np.zeros_like(c["beta"])
    dq, dk, dv, da, db, dS0 = _oracle(c, fn)
    S0 = c["S0"][0]
    want_dq = np.einsum("hkv,thv->thk", S0, c["dO"])
    want_dS0 = c["dST"][0] + np.einsum("thk,thv->hkv", c["q"], c["dO"])
    return (np.allclose(dq, want_dq, rtol=1e-12, atol=1e-12) and np.allclose(dS0[0], want_dS0, rtol=1e-12,
                                                                             atol=1e-12)
            and np.all(dk == 0) and np.all(dv == 0))


PINS = [pin_autograd, pin_finite_differences, pin_identity_closed_form]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    assert pin(bw.kda_backward)


def _mutant(edit):
    """The oracle's source with one planted edit, compiled fresh."""
    import inspect
    src = inspect.getsource(bw)
    old, new = edit
    assert old in src
    ns = {}
    exec(compile(src.replace(old, new), "mutant", "exec"), ns)
    return ns["kda_backward"]


MUTANTS = {
    "dq_from_previous_state": ('out["dq"][t] = np.einsum("hkv,hv->hk", St, dO[t])',
                               'out["dq"][t] = np.einsum("hkv,hv->hk", Sp, dO[t])'),
    "dk_without_recall_term": ('- np.einsum("hkv,hv->hk", X, gk))', '- 0.0 * np.einsum("hkv,hv->hk", X, gk))'),
    "no_decay_on_gradient": ("G = a[:, :, None] * E", "G = E"),
    "dalpha_from_unerased": ("da = np.sum(E * Sp, axis=2)", "da = np.sum(G * Sp, axis=2)"),
    "dv_without_beta": ('out["dv"][t] = beta[t][:, None] * gk', 'out["dv"][t] = gk'),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    fn = _mutant(MUTANTS[name])
    failed = [p.__name__ for p in PINS if not p(fn)]
    assert failed, f"no pin catches {name}"
