"""PyTorch-facing wrappers of the libslay C ABI.

Argument marshalling only: tensors supply device pointers and the current
HIP stream; every step of the computation runs in the HIP kernels behind
include/slay.h.  There is no CPU or PyTorch fallback -- if libslay.so is
missing or the tensors are not on a GPU the calls raise.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return _lib.SLAY_F32
    if t == torch.bfloat16:
        return _lib.SLAY_BF16
    raise TypeError(f"unsupported dtype {t} (float32 or bfloat16)")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    if not t.is_cuda:
        raise RuntimeError("libslay works on GPU tensors only")
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, shape=None, dtype=None) -> None:
    if not t.is_cuda:
        raise RuntimeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _need_d(t: torch.Tensor, name: str, d: int) -> None:
    """The last axis of q/k/x must be the draws' d (the kernels read d columns per row)."""
    if t.dim() < 1 or t.shape[-1] != d:
        raise ValueError(f"{name} has last dimension {t.shape[-1] if t.dim() else None}, the draws have d = {d}")


@dataclass
class FeatureMap:
    """Anchor and PRF draws plus the Gauss-Laguerre mixture settings.

    anchors, prf: [R*m, d] (one draw for every head) or [n_sets, R*m, d]
    (head h uses set h % n_sets), float32 or bfloat16, on the GPU.
    """

    anchors: torch.Tensor
    prf: torch.Tensor
    R: int
    m: int
    eps: float = 1e-3

    def __post_init__(self):
        _need(self.anchors, "anchors")
        _need(self.prf, "prf", tuple(self.anchors.shape), self.anchors.dtype)
        if self.anchors.shape[-2] != self.R * self.m:
            raise ValueError("draws must have R*m rows")
        self.n_sets = 1 if self.anchors.dim() == 2 else int(self.anchors.shape[0])
        self.d = int(self.anchors.shape[-1])
        self._c = _lib.SlayParams(self.d, self.R, self.m, float(self.eps), self.anchors.data_ptr(),
                                  self.prf.data_ptr(), _dtype_code(self.anchors.dtype), self.n_sets,
                                  self.R * self.m * self.d)

    @property
    def F(self) -> int:
        return self.R * self.m

    @property
    def dtype(self) -> torch.dtype:
        return self.anchors.dtype

    def c_params(self):
        return ctypes.byref(self._c)


def gl_table(R: int, eps: float):
    """The library's mixture parameters (alpha_r, beta_r), fp64 (host only)."""
    lib = _lib.load()
    a = (ctypes.c_double * R)()
    b = (ctypes.c_double * R)()
    _lib.check(lib.slay_gl_table(R, eps, a, b), "slay_gl_table")
    return np.array(a[:]), np.array(b[:])


def orthogonal_draws(n_rows: int, d: int, gauss: np.ndarray, chi: np.ndarray) -> np.ndarray:
    """Rows in orthogonal blocks of d, each marginally N(0, I_d), from the
    caller's Gaussian matrices gauss, chi [ceil(n_rows/d), d, d] (host, fp64);
    returns [n_rows, d] float32 on the host (slay_orthogonal_draws)."""
    lib = _lib.load()
    nb = (n_rows + d - 1) // d
    g = np.ascontiguousarray(gauss, dtype=np.float64)
    c = np.ascontiguousarray(chi, dtype=np.float64)
    if g.shape != (nb, d, d) or c.shape != (nb, d, d):
        raise ValueError(f"gauss and chi must be [{nb}, {d}, {d}]")
    out = np.empty((n_rows, d), dtype=np.float32)
    dp = ctypes.POINTER(ctypes.c_double)
    _lib.check(lib.slay_orthogonal_draws(n_rows, d, g.ctypes.data_as(dp), c.ctypes.data_as(dp),
                                         out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))), "slay_orthogonal_draws")
    return out


def featmap(fm: FeatureMap, x: torch.Tensor, out_dtype: torch.dtype | None = None,
            rows_per_head: int = 0, out: torch.Tensor | None = None) -> torch.Tensor:
    """phi(x) for rows x [..., d]; returns [..., R*m] in out_dtype (default x.dtype)."""
    lib = _lib.load()
    _need_d(x, "x", fm.d)
    _need(x, "x")
    out_dtype = out_dtype or x.dtype
    n = x.numel() // fm.d
    if out is None:
        out = torch.empty(x.shape[:-1] + (fm.F,), dtype=out_dtype, device=x.device)
    _need(out, "out", x.shape[:-1] + (fm.F,), out_dtype)
    phi = out
    st = lib.slay_featmap(fm.c_params(), x.data_ptr(), _dtype_code(x.dtype), n, rows_per_head, phi.data_ptr(),
                          _dtype_code(out_dtype), _stream(x))
    _lib.check(st, "slay_featmap")
    return phi


def chunked_fwd_workspace_size(fm: FeatureMap, B: int, H: int, L: int, dv: int, chunk: int,
                               dtype: torch.dtype) -> int:
    lib = _lib.load()
    return int(lib.slay_attn_chunked_fwd_workspace_size(fm.c_params(), B, H, L, dv, chunk, _dtype_code(dtype)))


def _fwd_outputs(fm: FeatureMap, q, k, v, S0, z0, return_state, out, S_out, z_out):
    """Validate the causal forward's tensors and create the outputs the caller did not pass."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d]")
    _need_d(q, "q", fm.d)
    _need(q, "q")
    B, H, L, _ = q.shape
    dv = v.shape[-1]
    _need(k, "k", q.shape, q.dtype)
    _need(v, "v", (B, H, L, dv), q.dtype)
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    _need(out, "out", (B, H, L, dv), q.dtype)
    for t, name, shp in ((S0, "S0", (B * H, fm.F, dv)), (z0, "z0", (B * H, fm.F))):
        if t is not None:
            _need(t, name, shp, torch.float32)
    if return_state:
        if S_out is None:
            S_out = torch.empty((B * H, fm.F, dv), dtype=torch.float32, device=q.device)
        if z_out is None:
            z_out = torch.empty((B * H, fm.F), dtype=torch.float32, device=q.device)
    for t, name, shp in ((S_out, "S_out", (B * H, fm.F, dv)), (z_out, "z_out", (B * H, fm.F))):
        if t is not None:
            _need(t, name, shp, torch.float32)
    return B, H, L, dv, out, S_out, z_out


def chunked_fwd(fm: FeatureMap, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, chunk: int,
                S0: torch.Tensor | None = None, z0: torch.Tensor | None = None, return_state: bool = False,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, S_out=None, z_out=None):
    """Causal SLAY forward.  q, k [B, H, L, d]; v [B, H, L, dv] -> o [B, H, L, dv].

    S0, z0: optional fp32 initial state [B*H, F, dv], [B*H, F].  With
    return_state the final state (S, z) is returned as well.
    """
    lib = _lib.load()
    B, H, L, dv, out, S_out, z_out = _fwd_outputs(fm, q, k, v, S0, z0, return_state, out, S_out, z_out)
    nbytes = chunked_fwd_workspace_size(fm, B, H, L, dv, chunk, q.dtype)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace")
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.slay_attn_chunked_fwd(fm.c_params(), q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q.dtype), B,
                                   H, L, dv, chunk, _ptr(S0), _ptr(z0), out.data_ptr(), _ptr(S_out), _ptr(z_out),
                                   _ptr(workspace), wsz, _stream(q))
    _lib.check(st, "slay_attn_chunked_fwd")
    if return_state:
        return out, S_out, z_out
    return out


def chunked_fwd_noalloc(fm: FeatureMap, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, chunk: int,
                        S0: torch.Tensor | None = None, z0: torch.Tensor | None = None, return_state: bool = False,
                        out: torch.Tensor | None = None, S_out=None, z_out=None):
    """chunked_fwd through slay_attn_chunked_fwd_noalloc: the library's fixed
    device scratch replaces the workspace, so the C call allocates nothing (the
    outputs are created here unless the caller passes them)."""
    lib = _lib.load()
    B, H, L, dv, out, S_out, z_out = _fwd_outputs(fm, q, k, v, S0, z0, return_state, out, S_out, z_out)
    st = lib.slay_attn_chunked_fwd_noalloc(fm.c_params(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           _dtype_code(q.dtype), B, H, L, dv, chunk, _ptr(S0), _ptr(z0),
                                           out.data_ptr(), _ptr(S_out), _ptr(z_out), _stream(q))
    _lib.check(st, "slay_attn_chunked_fwd_noalloc")
    if return_state:
        return out, S_out, z_out
    return out


def varlen_fwd_workspace_size(fm: FeatureMap, n_seqs: int, H: int, total_tokens: int, dv: int,
                              dtype: torch.dtype) -> int:
    lib = _lib.load()
    return int(lib.slay_attn_varlen_fwd_workspace_size(fm.c_params(), n_seqs, H, total_tokens, dv, _dtype_code(dtype)))


def varlen_fwd(fm: FeatureMap, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
               S0: torch.Tensor | None = None, z0: torch.Tensor | None = None, return_state: bool = False,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, S_out=None, z_out=None):
    """Causal SLAY forward over sequences of different lengths packed per head.

    q, k [H, T, d]; v [H, T, dv]; cu_seqlens int64 [n_seqs + 1] on the GPU
    (sequence s = tokens cu[s] .. cu[s+1] - 1 of every head) -> o [H, T, dv].
    S0, z0: optional fp32 initial states [n_seqs, H, F, dv], [n_seqs, H, F];
    with return_state the final states are returned as well.
    """
    lib = _lib.load()
    if q.dim() != 3:
        raise ValueError("q must be [H, T, d]")
    _need_d(q, "q", fm.d)
    _need(q, "q")
    H, T, _ = q.shape
    dv = v.shape[-1]
    n_seqs = cu_seqlens.numel() - 1
    _need(k, "k", q.shape, q.dtype)
    _need(v, "v", (H, T, dv), q.dtype)
    _need(cu_seqlens, "cu_seqlens", None, torch.int64)
    if out is None:
        out = torch.empty((H, T, dv), dtype=q.dtype, device=q.device)
    _need(out, "out", (H, T, dv), q.dtype)
    for t, name, shp in ((S0, "S0", (n_seqs, H, fm.F, dv)), (z0, "z0", (n_seqs, H, fm.F))):
        if t is not None:
            _need(t, name, shp, torch.float32)
    if return_state:
        if S_out is None:
            S_out = torch.empty((n_seqs, H, fm.F, dv), dtype=torch.float32, device=q.device)
        if z_out is None:
            z_out = torch.empty((n_seqs, H, fm.F), dtype=torch.float32, device=q.device)
    for t, name, shp in ((S_out, "S_out", (n_seqs, H, fm.F, dv)), (z_out, "z_out", (n_seqs, H, fm.F))):
        if t is not None:
            _need(t, name, shp, torch.float32)
    nbytes = varlen_fwd_workspace_size(fm, n_seqs, H, T, dv, q.dtype)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace")
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.slay_attn_varlen_fwd(fm.c_params(), q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q.dtype),
                                  n_seqs, H, cu_seqlens.data_ptr(), T, dv, _ptr(S0), _ptr(z0), out.data_ptr(),
                                  _ptr(S_out), _ptr(z_out), _ptr(workspace), wsz, _stream(q))
    _lib.check(st, "slay_attn_varlen_fwd")
    if return_state:
        return out, S_out, z_out
    return out


def chunked_bwd_workspace_size(fm: FeatureMap, B: int, H: int, L: int, dv: int, chunk: int,
                               dtype: torch.dtype) -> int:
    lib = _lib.load()
    return int(lib.slay_attn_chunked_bwd_workspace_size(fm.c_params(), B, H, L, dv, chunk, _dtype_code(dtype)))


def chunked_bwd(fm: FeatureMap, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor, chunk: int,
                S0: torch.Tensor | None = None, z0: torch.Tensor | None = None, dS_T: torch.Tensor | None = None,
                dz_T: torch.Tensor | None = None, state_grad: bool = False, workspace: torch.Tensor | None = None,
                dq=None, dk=None, dv=None, dS0=None, dz0=None):
    """Backward of chunked_fwd.  Given dout [B, H, L, dv] (and optionally the
    gradient of the final state dS_T [B*H, F, dv], dz_T [B*H, F]), returns
    (dq, dk, dv), plus (dS0, dz0) when state_grad is set."""
    lib = _lib.load()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d]")
    _need_d(q, "q", fm.d)
    _need(q, "q")
    B, H, L, _ = q.shape
    dvn = v.shape[-1]
    _need(k, "k", q.shape, q.dtype)
    _need(v, "v", (B, H, L, dvn), q.dtype)
    _need(dout, "dout", (B, H, L, dvn), q.dtype)
    for t, name, shp in ((S0, "S0", (B * H, fm.F, dvn)), (z0, "z0", (B * H, fm.F)),
                         (dS_T, "dS_T", (B * H, fm.F, dvn)), (dz_T, "dz_T", (B * H, fm.F))):
        if t is not None:
            _need(t, name, shp, torch.float32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", q.shape, q.dtype)
    _need(dk, "dk", q.shape, q.dtype)
    _need(dv, "dv", v.shape, q.dtype)
    if state_grad:
        if dS0 is None:
            dS0 = torch.empty((B * H, fm.F, dvn), dtype=torch.float32, device=q.device)
        if dz0 is None:
            dz0 = torch.empty((B * H, fm.F), dtype=torch.float32, device=q.device)
    for t, name, shp in ((dS0, "dS0", (B * H, fm.F, dvn)), (dz0, "dz0", (B * H, fm.F))):
        if t is not None:
            _need(t, name, shp, torch.float32)
    nbytes = chunked_bwd_workspace_size(fm, B, H, L, dvn, chunk, q.dtype)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace")
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.slay_attn_chunked_bwd(fm.c_params(), q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                   _dtype_code(q.dtype), B, H, L, dvn, chunk, _ptr(S0), _ptr(z0), _ptr(dS_T),
                                   _ptr(dz_T), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _ptr(dS0), _ptr(dz0),
                                   _ptr(workspace), wsz, _stream(q))
    _lib.check(st, "slay_attn_chunked_bwd")
    if state_grad:
        return dq, dk, dv, dS0, dz0
    return dq, dk, dv


def noncausal_fwd_workspace_size(fm: FeatureMap, B: int, H: int, Lq: int, Lk: int, dv: int,
                                 dtype: torch.dtype) -> int:
    lib = _lib.load()
    return int(lib.slay_attn_noncausal_fwd_workspace_size(fm.c_params(), B, H, Lq, Lk, dv, _dtype_code(dtype)))


def noncausal_fwd(fm: FeatureMap, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  S0: torch.Tensor | None = None, z0: torch.Tensor | None = None, return_state: bool = False,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, S_out=None, z_out=None):
    """Non-causal SLAY forward.  q [B, H, Lq, d]; k [B, H, Lk, d]; v [B, H, Lk, dv] -> o [B, H, Lq, dv].

    Every query attends to every key.  S0, z0: optional fp32 initial state
    [B*H, F, dv], [B*H, F].  With return_state the final state (S, z) is
    returned as well.
    """
    lib = _lib.load()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k must be [B, H, L, d]")
    _need_d(q, "q", fm.d)
    _need(q, "q")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    dv = v.shape[-1]
    _need(k, "k", (B, H, Lk, d), q.dtype)
    _need(v, "v", (B, H, Lk, dv), q.dtype)
    if out is None:
        out = torch.empty((B, H, Lq, dv), dtype=q.dtype, device=q.device)
    _need(out, "out", (B, H, Lq, dv), q.dtype)
    for t, name, shp in ((S0, "S0", (B * H, fm.F, dv)), (z0, "z0", (B * H, fm.F))):
        if t is not None:
            _need(t, name, shp, torch.float32)
    if return_state:
        if S_out is None:
            S_out = torch.empty((B * H, fm.F, dv), dtype=torch.float32, device=q.device)
        if z_out is None:
            z_out = torch.empty((B * H, fm.F), dtype=torch.float32, device=q.device)
    for t, name, shp in ((S_out, "S_out", (B * H, fm.F, dv)), (z_out, "z_out", (B * H, fm.F))):
        if t is not None:
            _need(t, name, shp, torch.float32)
    nbytes = noncausal_fwd_workspace_size(fm, B, H, Lq, Lk, dv, q.dtype)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace")
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.slay_attn_noncausal_fwd(fm.c_params(), q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q.dtype),
                                     B, H, Lq, Lk, dv, _ptr(S0), _ptr(z0), out.data_ptr(), _ptr(S_out),
                                     _ptr(z_out), _ptr(workspace), wsz, _stream(q))
    _lib.check(st, "slay_attn_noncausal_fwd")
    if return_state:
        return out, S_out, z_out
    return out


def recurrent_step_workspace_size(fm: FeatureMap, n_heads: int, dv: int, dtype: torch.dtype) -> int:
    lib = _lib.load()
    return int(lib.slay_attn_recurrent_step_workspace_size(fm.c_params(), n_heads, dv, _dtype_code(dtype)))


def recurrent_step(fm: FeatureMap, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, S: torch.Tensor,
                   z: torch.Tensor, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step for n heads: q, k [n, d], v [n, dv]; S [n, F, dv], z [n, F] fp32 in place."""
    lib = _lib.load()
    if q.dim() != 2:
        raise ValueError("q must be [n_heads, d]")
    _need_d(q, "q", fm.d)
    _need(q, "q")
    n = q.shape[0]
    dv = v.shape[-1]
    _need(k, "k", q.shape, q.dtype)
    _need(v, "v", (n, dv), q.dtype)
    _need(S, "S", (n, fm.F, dv), torch.float32)
    _need(z, "z", (n, fm.F), torch.float32)
    if out is None:
        out = torch.empty((n, dv), dtype=q.dtype, device=q.device)
    _need(out, "out", (n, dv), q.dtype)
    nbytes = recurrent_step_workspace_size(fm, n, dv, q.dtype)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace")
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.slay_attn_recurrent_step(fm.c_params(), q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q.dtype),
                                      n, dv, S.data_ptr(), z.data_ptr(), out.data_ptr(), _ptr(workspace), wsz,
                                      _stream(q))
    _lib.check(st, "slay_attn_recurrent_step")
    return out
