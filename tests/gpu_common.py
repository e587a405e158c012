"""Helpers shared by the GPU parity tests."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances: relative, per sequence (see seq_rel_err); fp32 storage of every
# input and output vs bf16 storage of b, c or y.
TOL_FP32 = 1e-4
TOL_BF16 = 2e-2


def tol_of(inp) -> float:
    return TOL_BF16 if (inp.bc_bf16 or inp.y_bf16) else TOL_FP32


def seq_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over elements of |got - ref| / (|ref| + rms(ref over the last axis)).

    The rms term keeps near-zero values of a sequence from dominating: a
    value is judged against its own size plus the typical size of its
    sequence (per (b,h) row of y, or per state vector of x_final).
    """
    got = np.asarray(got)
    ref = np.asarray(ref)
    rms = np.sqrt(np.mean(np.abs(ref) ** 2, axis=-1, keepdims=True))
    scale = np.abs(ref) + rms
    scale = np.where(scale == 0, 1.0, scale)
    return float(np.max(np.abs(got - ref) / scale)) if got.size else 0.0


def y_to_np(y: torch.Tensor) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)


def x_to_np(x: torch.Tensor, cplx: bool) -> np.ndarray:
    a = x.cpu().numpy().astype(np.float64)
    return a[..., 0] + 1j * a[..., 1] if cplx else a
