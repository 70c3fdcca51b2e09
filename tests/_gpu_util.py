"""Helpers shared by the GPU parity tests (device transfer, comparison, logging)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from megatron_tensor_transformer_gemm_amd import inputs as I

BF16_TOL = 2e-2   # normwise max relative error, bf16 inputs with fp32 accumulation
F32_TOL = 1e-5    # normwise max relative error, fp32 path

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Upload a generated tensor (bf16 bit patterns or float32) to cuda:0."""
    if dtype == I.BF16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda:0")


def host64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a device tensor (bf16 or fp32)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return I.as_f64(a, dtype)


def nerr(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (den if den > 0 else 1.0)


def sample_rows(T: int, k: int, seed: int) -> np.ndarray:
    """Seeded sample of k token rows, always including the first and the last."""
    g = np.random.default_rng(seed)
    rows = g.choice(T, size=min(k, T), replace=False)
    return np.unique(np.concatenate([[0, T - 1], rows]))
