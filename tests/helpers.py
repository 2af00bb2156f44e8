"""Shared helpers for the GPU parity tests (comparison metrics, tensor moves)."""
from __future__ import annotations

import numpy as np

# Parity bars: row-normwise max relative error (max over rows of
# |o_gpu - o_ref|_2 / |o_ref|_2), fp32 inputs 1e-4, bf16 inputs 2e-2.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rownorm_rel(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got.shape[-1]
    g = got.reshape(-1, d)
    r = ref.reshape(-1, d)
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    return float(np.max(num / np.maximum(den, 1e-300)))


def headnorm_rel(got, ref) -> float:
    """Max over heads (leading axis) of the relative Frobenius error of one head's array.

    Used for recurrent states after few tokens: a state row of feature f is
    then a handful of phi_f values, whose fp32 relative error is unbounded
    where (a.xh)^2 cancels (a nearly orthogonal to xh), so a per-row ratio is
    ill-posed the same way an elementwise one is; the head's whole state is
    the well-conditioned unit.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g = got.reshape(got.shape[0], -1)
    r = ref.reshape(ref.shape[0], -1)
    return float(np.max(np.linalg.norm(g - r, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-300)))


def elem_rel(got, ref, floor_frac=1e-3) -> float:
    """Elementwise relative error with a floor of floor_frac * rms(ref) (reported, not gated)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    floor = floor_frac * np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor)))


def to_dev(a, dtype: str):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def torch_dtype(dtype: str):
    import torch

    return torch.bfloat16 if dtype == "bf16" else torch.float32
