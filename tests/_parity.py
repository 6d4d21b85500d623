"""Shared helpers of the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np

# Tolerances of the path: bf16 outputs max-abs <= 1e-2 and rel-L2 <= 5e-3 against the fp64
# oracle; fp32 outputs 1e-5 for both.
TOL = {"bf16": (1e-2, 5e-3), "f32": (1e-5, 1e-5)}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def errors(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite output"
    d = gpu - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)) if d.size else 0.0
    return max_abs, rel


def assert_close(gpu, ref, dtype: str, what: str = ""):
    ma, rl = errors(gpu, ref)
    tol_abs, tol_rel = TOL[dtype]
    assert ma <= tol_abs and rl <= tol_rel, f"{what}: max-abs {ma:.3e} (tol {tol_abs}), rel-L2 {rl:.3e} (tol {tol_rel})"
    return ma, rl


def sample_rows(n: int, count: int, seed: int) -> np.ndarray:
    """Sorted sample of query rows that always includes the first, the last, tile edges and
    the ragged tail."""
    g = np.random.Generator(np.random.PCG64(seed))
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, n - 129, n - 65, n - 64, n - 33, n - 2, n - 1]
    rest = g.choice(n, size=min(count, n), replace=False)
    rows = np.unique(np.clip(np.concatenate([fixed, rest]), 0, n - 1))
    return rows
