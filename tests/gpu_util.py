"""Helpers for the GPU parity tests: seeded problems, device copies, and the
acceptance check against the fp64 oracle."""
from __future__ import annotations

import functools

import numpy as np

import oracle
import synth

REL_L2 = 1e-3      # per output row: ||y - y_ref|| / ||y_ref||
ELEM = 2e-3        # per element: |y - y_ref| <= ELEM * sum |w^| |xe|


def torch_dev():
    import torch
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=8)
def weights(j: int, N: int, K: int, sigma: float):
    return synth.quantized_weights(j, N, K, sigma)


@functools.lru_cache(maxsize=8)
def packed(j: int, N: int, K: int, sigma: float, max_batch: int = 16):
    from activation_sparse_bit_amd import sgemv
    q, s, z = weights(j, N, K, sigma)
    return sgemv.PackedMatrix(q, s, z, device=torch_dev(), max_batch=max_batch)


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch_dev())


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, B: np.ndarray, what: str = ""):
    """Acceptance: per-row relative L2 <= 1e-3 and every element within
    2e-3 * B of the oracle (B == 0 requires an exact zero)."""
    y = np.asarray(y_gpu, dtype=np.float64).reshape(y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - y_ref)
    bad = err > ELEM * B
    assert not bad.any(), (f"{what}: {bad.sum()} elements outside 2e-3*B; worst ratio "
                           f"{float((err / np.maximum(B, 1e-300)).max()):.3e} at "
                           f"{np.unravel_index(np.argmax(err - ELEM * B), err.shape)}")
    for m in range(y_ref.shape[0]):
        nr = np.linalg.norm(y_ref[m])
        if nr == 0:
            assert np.all(y[m] == 0), what
            continue
        rel = np.linalg.norm(y[m] - y_ref[m]) / nr
        assert rel <= REL_L2, f"{what}: row {m} rel L2 {rel:.3e}"
    return float(max((np.linalg.norm(y[m] - y_ref[m]) / max(np.linalg.norm(y_ref[m]), 1e-300))
                     for m in range(y_ref.shape[0])))


def sample_rows(N: int, n: int, seed: int = 0) -> np.ndarray:
    """Sorted sample of output rows that always includes the first and last
    row of every 512-row tile boundary pair and both ends of the matrix."""
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(N, size=min(n, N), replace=False).tolist())
    pick.update([0, N - 1, 511 % N, min(512, N - 1)])
    return np.array(sorted(pick))


def oracle_rows(q, s, z, x, t, rows):
    """Masked oracle restricted to a subset of output rows."""
    return oracle.gemv_masked(q[rows], s[rows], z[rows], x, t)
