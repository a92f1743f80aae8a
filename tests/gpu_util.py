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
