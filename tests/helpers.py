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


def rowfloor_rel(got, ref, heads: int = 1, floor_frac: float = 0.1) -> float:
    """Per-row relative error with a floor: max over rows i of
    |got_i - ref_i|_2 / max(|ref_i|_2, floor_frac * rms_i |ref_i|_2),
    the rms taken over the rows of the same head (the leading `heads` rows
    blocks of the flattened array, equal sizes).

    The gate for arrays whose rows can legitimately be tiny next to their
    neighbours: rows of a state after few tokens (a feature row holds a
    handful of phi values, each with the fp32 cancellation of (a.xh)^2 when a
    is nearly orthogonal to xh), or rows of dq, dk (the projection
    (I - xh xh^T) of a feature-space gradient nearly parallel to xh).  Such a
    row is measured against a tenth of the head's typical row, while every
    row of ordinary size -- and any row that is wholly wrong -- is held to the
    full relative bar.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got.shape[-1] if got.ndim > 1 else 1
    g = got.reshape(heads, -1, d)
    r = ref.reshape(heads, -1, d)
    num = np.linalg.norm(g - r, axis=2)
    den = np.linalg.norm(r, axis=2)
    rms = np.sqrt(np.mean(den * den, axis=1, keepdims=True))
    if num.size == 0:
        return 0.0
    return float(np.max(num / np.maximum(np.maximum(den, floor_frac * rms), 1e-300)))


def headnorm_rel(got, ref) -> float:
    """Max over heads (leading axis) of the relative Frobenius error of one head's array
    (reported beside the per-row gate; not a gate by itself)."""
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
