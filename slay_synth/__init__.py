"""Seeded synthetic inputs for causal SLAY workloads.

Shared by the tests, the smoke check and the benchmark; imported by both the
HIP path's tests and the oracle's tests.  It holds none of the method's
arithmetic: only Gaussian draws, the workload recipe's fp32 unit
normalisation of q and k, and fp32 -> bf16 round-to-nearest-even.

Recipe (the pages train on corpora and image/label sets that are not
available; these synthetic inputs stand in for them):
  q, k, v ~ i.i.d. N(0, 1) in fp32; q and k are then scaled to unit L2 norm
  in fp32 and, for bf16 workloads, rounded to bf16 (RNE).  The anchor and PRF
  draws are i.i.d. N(0, 1) of shape [R*m, d] (row r*m + t), rounded to bf16
  for bf16 workloads.  Seeds: inputs use ``default_rng([workload_id, 0])``,
  draws ``[workload_id, 1]``, decode step t ``[workload_id, 2, t]``, loss
gradients for the backward ``[workload_id, 3]``.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    B: int
    H: int
    L: int
    d: int
    dv: int
    R: int
    m: int
    chunk: int
    dtype: str  # "f32" or "bf16"
    eps: float = 1e-3
    steps: int = 0  # decode workloads: number of single-token steps

    @property
    def F(self) -> int:
        return self.R * self.m

    @property
    def n_heads(self) -> int:
        return self.B * self.H

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # tiny fp32 forward (parity only)
    "tiny_f32": Workload("tiny_f32", 1, B=1, H=1, L=256, d=64, dv=64, R=2, m=16, chunk=32, dtype="f32"),
    # B4 H8 L2048 bf16 forward
    "b4h8_l2k_bf16": Workload("b4h8_l2k_bf16", 2, B=4, H=8, L=2048, d=64, dv=64, R=3, m=32, chunk=64,
                              dtype="bf16"),
    # B1 H16 L16384 bf16 forward (the headline workload)
    "h16_l16k_bf16": Workload("h16_l16k_bf16", 3, B=1, H=16, L=16384, d=64, dv=64, R=4, m=64, chunk=64,
                              dtype="bf16"),
    # B1 H8 L131072 d=dv=128 bf16 forward
    "h8_l128k_d128_bf16": Workload("h8_l128k_d128_bf16", 4, B=1, H=8, L=131072, d=128, dv=128, R=4, m=128,
                                   chunk=128, dtype="bf16"),
    # recurrent decode: 256 sequences x 16 heads, 4096 single-token steps, fp32
    "decode_256x16_f32": Workload("decode_256x16_f32", 5, B=256, H=16, L=1, d=64, dv=64, R=4, m=64, chunk=1,
                                  dtype="f32", steps=4096),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).reshape(x.shape)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def orthogonal_gaussian_rows(rng, n: int, d: int) -> np.ndarray:
    """n rows in consecutive blocks of d mutually orthogonal directions.

    Each block is a Haar-random orthogonal matrix (QR of a Gaussian matrix
    with the signs of R's diagonal folded in), each row scaled by an
    independent chi(d) length, so every row is still marginally N(0, I_d)
    while the rows of a block are orthogonal: the "positive orthogonal random
    features" of the linearized 2-simplicial attention page's summary.
    """
    blocks = []
    for _ in range((n + d - 1) // d):
        Q, R = np.linalg.qr(rng.standard_normal((d, d)))
        Q = Q * np.sign(np.diag(R))
        lengths = np.linalg.norm(rng.standard_normal((d, d)), axis=1)
        blocks.append(Q.T * lengths[:, None])
    return np.concatenate(blocks)[:n]


def make_draws(w: Workload, seed=None, orthogonal: bool = False):
    """Anchor and PRF draws, each [R*m, d] fp32 (bf16-exact for bf16 workloads).

    orthogonal: the PRF rows of every node come in orthogonal blocks of d
    (orthogonal_gaussian_rows); anchors stay i.i.d. N(0, I).
    """
    rng = np.random.default_rng([w.wid, 1] if seed is None else seed)
    a = rng.standard_normal((w.F, w.d), dtype=np.float32)
    if orthogonal:
        g = np.concatenate([orthogonal_gaussian_rows(rng, w.m, w.d) for _ in range(w.R)]).astype(np.float32)
    else:
        g = rng.standard_normal((w.F, w.d), dtype=np.float32)
    return _finish(a, w.dtype), _finish(g, w.dtype)


def make_qkv(w: Workload, seed=None, near_pairs=None, qk_scale=None, zero_k=()):
    """q, k [B, H, L, d] and v [B, H, L, dv] fp32 (bf16-exact for bf16 workloads).

    The defaults give the workload recipe (q, k on the unit sphere).  Stress
    options, each drawn from its own seeded stream so the default arrays do
    not change:
      near_pairs = (u_lo, u_hi): every k_i is rebuilt as u_i q_i + sqrt(1-u_i^2) e_i
          with e_i a unit vector orthogonal to q_i and u_i ~ U(u_lo, u_hi), so
          q_i . k_i = u_i (up to rounding) -- the high-alignment set;
      qk_scale = (lo, hi): each q and k row is then multiplied by its own
          log-uniform factor in [lo, hi] (rows off the unit sphere);
      zero_k: token indices whose k rows are set to exactly zero.
    """
    base = [w.wid, 0] if seed is None else seed
    base = list(base) if isinstance(base, (list, tuple)) else [int(base)]
    rng = np.random.default_rng(base)
    shp = (w.B, w.H, w.L)
    q = rng.standard_normal(shp + (w.d,), dtype=np.float32)
    k = rng.standard_normal(shp + (w.d,), dtype=np.float32)
    v = rng.standard_normal(shp + (w.dv,), dtype=np.float32)
    q = _unit_rows(q)
    if near_pairs is not None:
        lo, hi = near_pairs
        r2 = np.random.default_rng(base + [101])
        u = r2.uniform(lo, hi, shp + (1,)).astype(np.float64)
        q64 = q.astype(np.float64)
        e = k.astype(np.float64)
        e = e - np.sum(e * q64, axis=-1, keepdims=True) * q64
        e = e / np.linalg.norm(e, axis=-1, keepdims=True)
        k = (u * q64 + np.sqrt(1.0 - u * u) * e).astype(np.float32)
    k = _unit_rows(k)
    if qk_scale is not None:
        lo, hi = qk_scale
        r3 = np.random.default_rng(base + [102])
        sq = np.exp(r3.uniform(np.log(lo), np.log(hi), shp + (1,))).astype(np.float32)
        sk = np.exp(r3.uniform(np.log(lo), np.log(hi), shp + (1,))).astype(np.float32)
        q = q * sq
        k = k * sk
    if len(zero_k):
        k[:, :, np.asarray(zero_k, dtype=np.int64)] = 0.0
    return _finish(q, w.dtype), _finish(k, w.dtype), _finish(v, w.dtype)


def make_decode_step(w: Workload, t: int, n_heads: int | None = None, qk_scale=None):
    """Single-token q, k [n_heads, d] and v [n_heads, dv] for decode step t (fp32).

    qk_scale = (lo, hi) multiplies each q and k row by its own log-uniform
    factor in [lo, hi] (drawn from a separate stream; the default arrays are
    unchanged)."""
    nh = w.n_heads if n_heads is None else n_heads
    rng = np.random.default_rng([w.wid, 2, int(t)])
    q = rng.standard_normal((nh, w.d), dtype=np.float32)
    k = rng.standard_normal((nh, w.d), dtype=np.float32)
    v = rng.standard_normal((nh, w.dv), dtype=np.float32)
    q, k = _unit_rows(q), _unit_rows(k)
    if qk_scale is not None:
        lo, hi = qk_scale
        r3 = np.random.default_rng([w.wid, 2, int(t), 102])
        q = q * np.exp(r3.uniform(np.log(lo), np.log(hi), (nh, 1))).astype(np.float32)
        k = k * np.exp(r3.uniform(np.log(lo), np.log(hi), (nh, 1))).astype(np.float32)
    return _finish(q, w.dtype), _finish(k, w.dtype), _finish(v, w.dtype)


def make_grads(w: Workload, seed=None):
    """Loss gradients for the backward: dout [B, H, L, dv] ~ N(0, 1) (bf16-exact
    for bf16 workloads) and final-state gradients dS_T [B*H, F, dv],
    dz_T [B*H, F] ~ N(0, 1) in fp32."""
    rng = np.random.default_rng([w.wid, 3] if seed is None else seed)
    dout = rng.standard_normal((w.B, w.H, w.L, w.dv), dtype=np.float32)
    dS = rng.standard_normal((w.n_heads, w.F, w.dv), dtype=np.float32)
    dz = rng.standard_normal((w.n_heads, w.F), dtype=np.float32)
    return _finish(dout, w.dtype), dS, dz
