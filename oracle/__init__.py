"""fp64 CPU oracle for causal SLAY attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it shares no code
with that path.  The arithmetic lives in ``slay_oracle.c``; this module only
builds that file with gcc and marshals numpy arrays into it.

Sources: "SLAY: Geometry-Aware Spherical Linearized Attention with
Yat-Kernel" (arXiv 2602.04915 abstract, paperdance page) and the nubint.ai
review of that paper ("Proposed method" bullets 1-6).  Each C function cites
the passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "slay_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile slay_oracle.c with gcc (fp64, IEEE semantics, OpenMP)."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.orc_gauss_laguerre.argtypes = [ctypes.c_int, _D, _D]
        lib.orc_node_params.argtypes = [ctypes.c_int, ctypes.c_double, _D, _D]
        lib.orc_yat_kernel.argtypes = [_I64, _D, ctypes.c_double, _D]
        lib.orc_yat_kernel.restype = None
        lib.orc_yat_mixture.argtypes = [_I64, _D, ctypes.c_double, ctypes.c_int, _D]
        lib.orc_featmap.argtypes = [_I64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                    _D, _D, _D, _D]
        lib.orc_attn_brute.argtypes = [_I64, ctypes.c_int, ctypes.c_int, _D, _D, _D, _D, _D, _D]
        lib.orc_attn_brute.restype = None
        lib.orc_attn_recurrent.argtypes = [_I64, ctypes.c_int, ctypes.c_int, _D, _D, _D, _D, _D, _D]
        lib.orc_attn_recurrent.restype = None
        lib.orc_attn_chunked.argtypes = [_I64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _D, _D, _D,
                                         _D, _D, _D]
        lib.orc_attn_chunked.restype = None
        lib.orc_slay_causal.argtypes = [_I64, _I64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_double, _D, _D, _D, _D, _D, _I64,
                                        ctypes.c_int, ctypes.c_int, _D, _D, _D, _D, _D]
        lib.orc_yat_exact_causal.argtypes = [_I64, _I64, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                             _D, _D, _D, _D]
        lib.orc_attn_rows.argtypes = [_I64, ctypes.POINTER(ctypes.c_int64), ctypes.c_int, ctypes.c_int,
                                      _D, _D, _D, _D]
        lib.orc_attn_rows.restype = None
        lib.orc_slay_noncausal.argtypes = [_I64, _I64, _I64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_double, _D, _D, _D, _D, _D, _I64, _D, _D,
                                           _D, _D, _D]
        lib.orc_featmap_vjp.argtypes = [_I64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                        _D, _D, _D, _D, _D]
        lib.orc_slay_causal_bwd.argtypes = [_I64, _I64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_double, _D, _D, _D, _D, _D, _I64, ctypes.c_int, _D, _D, _D,
                                            _D, _D, _D, _D, _D, _D, _D]
        lib.orc_max_threads.argtypes = []
        lib.orc_max_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(_D)


def _check(status: int, what: str) -> None:
    if status != 0:
        raise ValueError(f"oracle {what} rejected its arguments (status {status})")


def max_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_max_threads())


# --------------------------------------------------------------------------
def gauss_laguerre(R: int):
    """R-point Gauss-Laguerre nodes x and weights w (weight e^{-x} on [0, inf))."""
    lib = _load()
    x = np.zeros(R)
    w = np.zeros(R)
    _check(lib.orc_gauss_laguerre(int(R), _p(x), _p(w)), "gauss_laguerre")
    return x, w


def node_params(R: int, eps: float):
    """Mixture node parameters (alpha_r, beta_r) = (w_r/(2+eps), 2 x_r/(2+eps))."""
    lib = _load()
    a = np.zeros(R)
    b = np.zeros(R)
    _check(lib.orc_node_params(int(R), float(eps), _p(a), _p(b)), "node_params")
    return a, b


def yat_kernel(u, eps: float) -> np.ndarray:
    """Spherical Yat kernel K(u) = u^2/(2-2u+eps)."""
    lib = _load()
    u = _f64(u)
    out = np.zeros_like(u)
    lib.orc_yat_kernel(u.size, _p(u), float(eps), _p(out))
    return out


def yat_mixture(u, eps: float, R: int) -> np.ndarray:
    """Gauss-Laguerre discretisation K_R(u) = sum_r alpha_r u^2 exp(beta_r u)."""
    lib = _load()
    u = _f64(u)
    out = np.zeros_like(u)
    _check(lib.orc_yat_mixture(u.size, _p(u), float(eps), int(R), _p(out)), "yat_mixture")
    return out


def featmap(x, anchors, prf, eps: float, R: int, m: int) -> np.ndarray:
    """SLAY features phi(x) [n, R*m] of rows x [n, d]; draws [R*m, d] (or [R, m, d])."""
    lib = _load()
    x = _f64(x)
    d = x.shape[-1]
    x2 = x.reshape(-1, d)
    a = _f64(anchors).reshape(R * m, d)
    g = _f64(prf).reshape(R * m, d)
    out = np.zeros((x2.shape[0], R * m))
    _check(lib.orc_featmap(x2.shape[0], d, int(R), int(m), float(eps), _p(x2), _p(a), _p(g), _p(out)),
           "featmap")
    return out.reshape(x.shape[:-1] + (R * m,))


def attn_brute(phq, phk, v, S0=None, z0=None) -> np.ndarray:
    """Masked L x L normalised attention on features of one head."""
    lib = _load()
    phq, phk, v = _f64(phq), _f64(phk), _f64(v)
    L, F = phq.shape
    dv = v.shape[1]
    S0 = None if S0 is None else _f64(S0)
    z0 = None if z0 is None else _f64(z0)
    o = np.zeros((L, dv))
    lib.orc_attn_brute(L, F, dv, _p(phq), _p(phk), _p(v), _p(S0), _p(z0), _p(o))
    return o


def attn_recurrent(phq, phk, v, S=None, z=None):
    """Recurrent form of one head; returns (o, S_final, z_final)."""
    lib = _load()
    phq, phk, v = _f64(phq), _f64(phk), _f64(v)
    L, F = phq.shape
    dv = v.shape[1]
    S = np.zeros((F, dv)) if S is None else _f64(S).copy()
    z = np.zeros(F) if z is None else _f64(z).copy()
    o = np.zeros((L, dv))
    lib.orc_attn_recurrent(L, F, dv, _p(phq), _p(phk), _p(v), _p(S), _p(z), _p(o))
    return o, S, z


def attn_chunked(phq, phk, v, C: int, S=None, z=None):
    """Chunked form of one head (chunk C); returns (o, S_final, z_final)."""
    lib = _load()
    phq, phk, v = _f64(phq), _f64(phk), _f64(v)
    L, F = phq.shape
    dv = v.shape[1]
    S = np.zeros((F, dv)) if S is None else _f64(S).copy()
    z = np.zeros(F) if z is None else _f64(z).copy()
    o = np.zeros((L, dv))
    lib.orc_attn_chunked(L, F, dv, int(C), _p(phq), _p(phk), _p(v), _p(S), _p(z), _p(o))
    return o, S, z


FORMS = {"brute": 0, "recurrent": 1, "chunked": 2}


def slay_causal(q, k, v, anchors, prf, eps: float, R: int, m: int, form: str = "recurrent",
                chunk: int = 64, S0=None, z0=None, per_head_draws: bool = False):
    """Causal SLAY forward over heads.

    q, k: [..., L, d]; v: [..., L, dv] (leading dims are heads).  Draws are
    [R*m, d] shared by all heads, or [nh, R*m, d] when per_head_draws.
    Returns (o [..., L, dv], S [nh, F, dv], z [nh, F]).
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    L, d = q.shape[-2:]
    dv = v.shape[-1]
    nh = int(np.prod(lead)) if lead else 1
    F = R * m
    a = _f64(anchors)
    g = _f64(prf)
    stride = F * d if per_head_draws else 0
    if per_head_draws:
        assert a.size == nh * F * d and g.size == nh * F * d
    else:
        assert a.size == F * d and g.size == F * d
    S0p = None if S0 is None else _f64(S0).reshape(nh, F, dv)
    z0p = None if z0 is None else _f64(z0).reshape(nh, F)
    o = np.zeros(lead + (L, dv))
    S = np.zeros((nh, F, dv))
    z = np.zeros((nh, F))
    _check(lib.orc_slay_causal(nh, L, d, dv, int(R), int(m), float(eps), _p(q), _p(k), _p(v), _p(a),
                               _p(g), stride, FORMS[form], int(chunk), _p(S0p), _p(z0p), _p(o), _p(S),
                               _p(z)), "slay_causal")
    return o, S, z


def slay_noncausal(q, k, v, anchors, prf, eps: float, R: int, m: int, S0=None, z0=None,
                   per_head_draws: bool = False):
    """Non-causal SLAY over heads: every query attends to every key.

    q: [..., Lq, d]; k: [..., Lk, d]; v: [..., Lk, dv] (same leading dims).
    Returns (o [..., Lq, dv], S [nh, F, dv], z [nh, F]) with S, z the final
    state (S0, z0 plus every key).
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    Lq, d = q.shape[-2:]
    Lk = k.shape[-2]
    dv = v.shape[-1]
    nh = int(np.prod(lead)) if lead else 1
    F = R * m
    a = _f64(anchors)
    g = _f64(prf)
    stride = F * d if per_head_draws else 0
    if per_head_draws:
        assert a.size == nh * F * d and g.size == nh * F * d
    else:
        assert a.size == F * d and g.size == F * d
    S0p = None if S0 is None else _f64(S0).reshape(nh, F, dv)
    z0p = None if z0 is None else _f64(z0).reshape(nh, F)
    o = np.zeros(lead + (Lq, dv))
    S = np.zeros((nh, F, dv))
    z = np.zeros((nh, F))
    _check(lib.orc_slay_noncausal(nh, Lq, Lk, d, dv, int(R), int(m), float(eps), _p(q), _p(k), _p(v), _p(a),
                                  _p(g), stride, _p(S0p), _p(z0p), _p(o), _p(S), _p(z)), "slay_noncausal")
    return o, S, z


def yat_exact_causal(q, k, v, eps: float) -> np.ndarray:
    """Exact spherical-Yat causal attention (the quadratic comparison point)."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    L, d = q.shape[-2:]
    dv = v.shape[-1]
    nh = int(np.prod(lead)) if lead else 1
    o = np.zeros(lead + (L, dv))
    _check(lib.orc_yat_exact_causal(nh, L, d, dv, float(eps), _p(q), _p(k), _p(v), _p(o)),
           "yat_exact_causal")
    return o


def mean_kernel_closed_form(u, eps: float, R: int) -> np.ndarray:
    """E over draws of phi(q).phi(k) for unit q, k with q.k = u.

    Each node contributes (alpha_r/m) * m * E[(a.q)^2 (a.k)^2] * E[prf(q) prf(k)]
    = alpha_r (1 + 2u^2) exp(beta_r u): the first factor by Isserlis' theorem
    for a ~ N(0, I), the second by the Gaussian moment generating function.
    """
    alpha, beta = node_params(R, eps)
    u = _f64(u)
    return (1.0 + 2.0 * u * u) * sum(alpha[r] * np.exp(beta[r] * u) for r in range(R))


def attn_rows(rows, phq_rows, phk, v) -> np.ndarray:
    """Causal attention outputs of the selected rows of one head, each summed on its own."""
    lib = _load()
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    phq_rows, phk, v = _f64(phq_rows), _f64(phk), _f64(v)
    F = phk.shape[1]
    dv = v.shape[1]
    assert phq_rows.shape == (rows.size, F)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < phk.shape[0] and phk.shape[0] == v.shape[0])
    o = np.zeros((rows.size, dv))
    lib.orc_attn_rows(rows.size, rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), F, dv, _p(phq_rows),
                      _p(phk), _p(v), _p(o))
    return o


def featmap_vjp(x, anchors, prf, dphi, eps: float, R: int, m: int) -> np.ndarray:
    """dx = J_phi(x)^T dphi for rows x [n, d] (the feature map's backward)."""
    lib = _load()
    x = _f64(x)
    d = x.shape[-1]
    x2 = x.reshape(-1, d)
    a = _f64(anchors).reshape(R * m, d)
    g = _f64(prf).reshape(R * m, d)
    dphi = _f64(dphi).reshape(x2.shape[0], R * m)
    out = np.zeros_like(x2)
    _check(lib.orc_featmap_vjp(x2.shape[0], d, int(R), int(m), float(eps), _p(x2), _p(a), _p(g), _p(dphi),
                               _p(out)), "featmap_vjp")
    return out.reshape(x.shape)


BWD_FORMS = {"brute": 0, "recurrent": 1}


def slay_causal_bwd(q, k, v, dout, anchors, prf, eps: float, R: int, m: int, form: str = "recurrent",
                    S0=None, z0=None, dS_T=None, dz_T=None, per_head_draws: bool = False):
    """Backward of the causal SLAY forward over heads.

    dout: [..., L, dv], the loss gradient with respect to o; dS_T [nh, F, dv],
    dz_T [nh, F] (optional): with respect to the final state.
    Returns (dq, dk, dv, dS0 [nh, F, dv], dz0 [nh, F]).
    """
    lib = _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    lead = q.shape[:-2]
    L, d = q.shape[-2:]
    dv = v.shape[-1]
    nh = int(np.prod(lead)) if lead else 1
    F = R * m
    a = _f64(anchors)
    g = _f64(prf)
    stride = F * d if per_head_draws else 0
    if per_head_draws:
        assert a.size == nh * F * d and g.size == nh * F * d
    else:
        assert a.size == F * d and g.size == F * d
    assert dout.shape == v.shape
    opt = lambda t, shape: None if t is None else _f64(t).reshape(shape)
    S0p, z0p = opt(S0, (nh, F, dv)), opt(z0, (nh, F))
    dSTp, dzTp = opt(dS_T, (nh, F, dv)), opt(dz_T, (nh, F))
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dvv = np.zeros(v.shape)
    dS0 = np.zeros((nh, F, dv))
    dz0 = np.zeros((nh, F))
    _check(lib.orc_slay_causal_bwd(nh, L, d, dv, int(R), int(m), float(eps), _p(q), _p(k), _p(v), _p(a), _p(g),
                                   stride, BWD_FORMS[form], _p(S0p), _p(z0p), _p(dout), _p(dSTp), _p(dzTp),
                                   _p(dq), _p(dk), _p(dvv), _p(dS0), _p(dz0)), "slay_causal_bwd")
    return dq, dk, dvv, dS0, dz0


def slay_causal_varlen(q, k, v, cu_seqlens, anchors, prf, eps: float, R: int, m: int, S0=None, z0=None,
                       form: str = "recurrent"):
    """Causal SLAY over sequences packed along the token axis of every head.

    q, k: [H, T, d]; v: [H, T, dv]; cu_seqlens: [n_seqs + 1] offsets (sequence
    s = tokens cu[s] .. cu[s+1] - 1 of each head); S0, z0: optional initial
    states [n_seqs, H, F, dv], [n_seqs, H, F].  Each sequence is its own causal
    problem, started from its own state.  Returns (o [H, T, dv],
    S [n_seqs, H, F, dv], z [n_seqs, H, F]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    H, T, _ = q.shape
    dv = v.shape[-1]
    F = R * m
    n = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T and all(b <= e for b, e in zip(cu[:-1], cu[1:]))
    o = np.zeros((H, T, dv))
    S = np.zeros((n, H, F, dv))
    z = np.zeros((n, H, F))
    for s in range(n):
        b, e = cu[s], cu[s + 1]
        o_s, S_s, z_s = slay_causal(q[:, b:e], k[:, b:e], v[:, b:e], anchors, prf, eps, R, m, form=form,
                                    S0=None if S0 is None else _f64(S0)[s], z0=None if z0 is None else _f64(z0)[s])
        o[:, b:e] = o_s
        S[s], z[s] = S_s, z_s
    return o, S, z
