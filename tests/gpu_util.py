"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

import sys

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")


def announce(msg: str):
    """Name the case before a GPU step, flushed, so a fault can be attributed."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()
