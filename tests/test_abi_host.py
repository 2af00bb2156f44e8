"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every function include/slay.h declares, build
the same Gauss-Laguerre mixture the oracle does, and reject bad arguments on
the host with a status code and a message before any work is enqueued.
"""
import ctypes
import os
import re

import numpy as np
import pytest
from numpy.polynomial import laguerre as npl

from kernelized_linear_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_function(lib):
    hdr = open(os.path.join(ROOT, "include", "slay.h")).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(slay_\w+)\s*\(", hdr, flags=re.M))
    assert declared == set(_lib.EXPORTS), declared ^ set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.slay_version() == 100
    assert lib.slay_status_string(0) == b"ok"
    assert lib.slay_status_string(3) == b"device error"


@pytest.mark.parametrize("R", [1, 2, 3, 4, 8, 16])
def test_gl_table_matches_library_rule_and_oracle(lib, orc, R):
    eps = 1e-3
    a = (ctypes.c_double * R)()
    b = (ctypes.c_double * R)()
    assert lib.slay_gl_table(R, eps, a, b) == 0
    x, w = npl.laggauss(R)
    np.testing.assert_allclose(np.array(a[:]) * (2 + eps), w, rtol=1e-12)
    np.testing.assert_allclose(np.array(b[:]) * (2 + eps) / 2, x, rtol=1e-13)
    oa, ob = orc.node_params(R, eps)
    np.testing.assert_allclose(a[:], oa, rtol=1e-12)
    np.testing.assert_allclose(b[:], ob, rtol=1e-13)


def test_gl_table_rejects(lib):
    a = (ctypes.c_double * 20)()
    assert lib.slay_gl_table(0, 1e-3, a, a) == _lib.SLAY_E_INVALID
    assert lib.slay_gl_table(17, 1e-3, a, a) == _lib.SLAY_E_INVALID
    assert lib.slay_gl_table(2, 0.0, a, a) == _lib.SLAY_E_INVALID
    assert lib.slay_gl_table(2, 1e-3, None, a) == _lib.SLAY_E_INVALID
    assert b"R in [1, 16]" in lib.slay_last_error()


FAKE = 0x10000  # 16-byte aligned stand-in pointer: every case below fails before any launch


def _params(d=64, R=4, m=64, eps=1e-3, dt=_lib.SLAY_BF16, sets=1, stride=0, anchors=FAKE, prf=FAKE):
    return _lib.SlayParams(d, R, m, eps, anchors, prf, dt, sets, stride)


def _fwd(lib, p, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, dt=_lib.SLAY_BF16, B=1, H=16, L=16384, dv=64, chunk=64, S0=None, z0=None,
                o=FAKE, S_out=None, z_out=None, ws=None, ws_bytes=0)
    args.update(kw)
    return lib.slay_attn_chunked_fwd(ctypes.byref(p) if p is not None else None, args["q"], args["k"], args["v"],
                                     args["dt"], args["B"], args["H"], args["L"], args["dv"], args["chunk"],
                                     args["S0"], args["z0"], args["o"], args["S_out"], args["z_out"], args["ws"],
                                     args["ws_bytes"], None)


def test_chunked_fwd_validation(lib):
    E_INV, E_UNS = _lib.SLAY_E_INVALID, _lib.SLAY_E_UNSUPPORTED
    assert _fwd(lib, None) == E_INV
    assert _fwd(lib, _params(d=48)) == E_UNS
    assert _fwd(lib, _params(R=0)) == E_INV
    assert _fwd(lib, _params(m=24)) == E_UNS
    assert _fwd(lib, _params(eps=0.0)) == E_INV
    assert _fwd(lib, _params(eps=float("nan"))) == E_INV
    assert _fwd(lib, _params(anchors=None)) == E_INV
    assert _fwd(lib, _params(prf=FAKE + 2)) == E_INV  # misaligned draws
    assert _fwd(lib, _params(sets=2, stride=10)) == E_INV
    assert _fwd(lib, _params(), chunk=0) == E_INV
    assert _fwd(lib, _params(), chunk=129) == E_INV
    assert _fwd(lib, _params(), L=-1) == E_INV
    assert _fwd(lib, _params(), dv=0) == E_INV
    assert _fwd(lib, _params(), dt=_lib.SLAY_F32) == E_UNS  # io dtype must equal the draw dtype
    assert _fwd(lib, _params(), q=None) == E_INV
    assert _fwd(lib, _params(), o=FAKE + 4) == E_INV  # misaligned output
    assert _fwd(lib, _params(), dv=12) == E_UNS  # rows not whole 16-byte vectors
    assert b"workspace too small" in (lib.slay_last_error() if _fwd(lib, _params()) == E_INV else b"")
    need = lib.slay_attn_chunked_fwd_workspace_size(ctypes.byref(_params()), 1, 16, 16384, 64, 64, _lib.SLAY_BF16)
    assert need > 0
    assert _fwd(lib, _params(), ws=None, ws_bytes=need) == E_INV  # NULL workspace
    assert _fwd(lib, _params(), ws=FAKE + 8, ws_bytes=need) == E_INV  # misaligned workspace
    assert _fwd(lib, _params(), B=2 ** 31 - 1, H=2 ** 31 - 1, L=2 ** 40) == E_INV  # overflow


def test_workspace_sizes(lib):
    p = _params()
    # fused path: per-segment states, n_seg = 16 segments of 1024 tokens for 16 heads
    n = lib.slay_attn_chunked_fwd_workspace_size(ctypes.byref(p), 1, 16, 16384, 64, 64, _lib.SLAY_BF16)
    assert n == 4 * 16 * 16 * 256 * (64 + 16)
    # many heads: one segment, no workspace
    assert lib.slay_attn_chunked_fwd_workspace_size(ctypes.byref(p), 64, 16, 2048, 64, 64, _lib.SLAY_BF16) == 0
    # general path (fp32): phi(q), phi(k) and per-chunk states
    p32 = _params(R=2, m=16, dt=_lib.SLAY_F32)
    n = lib.slay_attn_chunked_fwd_workspace_size(ctypes.byref(p32), 1, 1, 256, 64, 32, _lib.SLAY_F32)
    assert n == 4 * (2 * 256 * 32 + 8 * 32 * 65)
    assert lib.slay_attn_chunked_fwd_workspace_size(ctypes.byref(p), 1, 16, 0, 64, 64, _lib.SLAY_BF16) == 0


def test_wide_path_workspace(lib):
    """bf16 shapes the fused kernels do not cover take the wide path: phi(q) and
    phi(k) in bf16 (256-byte aligned each) plus one fp32 state of F x (dv+16)
    per (head, segment), segments of whole 32-token chunks, about 256 of them
    over the batch."""
    r256 = lambda x: (x + 255) // 256 * 256
    p = _params(d=128, R=4, m=128)
    # B1 H8 L131072 d=dv=128 F=512, chunk 128: segments of 4096 tokens, 32 per head
    n = lib.slay_attn_chunked_fwd_workspace_size(ctypes.byref(p), 1, 8, 131072, 128, 128, _lib.SLAY_BF16)
    assert n == 2 * r256(8 * 131072 * 512 * 2) + 4 * 8 * 32 * 512 * 144
    # a short ragged sequence: segments of one chunk (32 tokens), ceil(1000 / 32) = 32 of them
    n = lib.slay_attn_chunked_fwd_workspace_size(ctypes.byref(p), 1, 2, 1000, 128, 32, _lib.SLAY_BF16)
    assert n == 2 * r256(2 * 1000 * 512 * 2) + 4 * 2 * 32 * 512 * 144
    # dv = 64 with F = 256 at chunk 32 (the fused kernels need chunk 64): 32-token segments, 32 per head
    p64 = _params(R=4, m=64)
    n = lib.slay_attn_chunked_fwd_workspace_size(ctypes.byref(p64), 1, 3, 1000, 64, 32, _lib.SLAY_BF16)
    assert n == 2 * r256(3 * 1000 * 256 * 2) + 4 * 3 * 32 * 256 * 80
    # F = 96 has no wide variant: the general path (fp32 phi and per-chunk states)
    p96 = _params(R=3, m=32)
    n = lib.slay_attn_chunked_fwd_workspace_size(ctypes.byref(p96), 1, 1, 500, 64, 32, _lib.SLAY_BF16)
    assert n == 4 * (2 * 500 * 96 + 16 * 96 * 65)


def test_featmap_and_decode_validation(lib):
    p = _params()
    assert lib.slay_featmap(None, FAKE, _lib.SLAY_BF16, 10, 0, FAKE, _lib.SLAY_BF16, None) == _lib.SLAY_E_INVALID
    assert lib.slay_featmap(ctypes.byref(p), FAKE, _lib.SLAY_F32, 10, 0, FAKE, _lib.SLAY_BF16, None) == \
        _lib.SLAY_E_UNSUPPORTED
    assert lib.slay_featmap(ctypes.byref(p), None, _lib.SLAY_BF16, 10, 0, FAKE, _lib.SLAY_BF16, None) == \
        _lib.SLAY_E_INVALID
    assert lib.slay_featmap(ctypes.byref(p), FAKE, _lib.SLAY_BF16, -1, 0, FAKE, _lib.SLAY_BF16, None) == \
        _lib.SLAY_E_INVALID
    assert lib.slay_featmap(ctypes.byref(p), FAKE, _lib.SLAY_BF16, 0, 0, FAKE, _lib.SLAY_BF16, None) == _lib.SLAY_OK
    ps = _params(sets=2, stride=4 * 64 * 64)
    assert lib.slay_featmap(ctypes.byref(ps), FAKE, _lib.SLAY_BF16, 10, 3, FAKE, _lib.SLAY_BF16, None) == \
        _lib.SLAY_E_INVALID  # rows_per_head must divide n_rows
    # decode
    pd = _params(dt=_lib.SLAY_F32)
    need = lib.slay_attn_recurrent_step_workspace_size(ctypes.byref(pd), 10, 64, _lib.SLAY_F32)
    assert need == 2 * 10 * 256 * 4
    st = lib.slay_attn_recurrent_step(ctypes.byref(pd), FAKE, FAKE, FAKE, _lib.SLAY_F32, 10, 64, None, FAKE, FAKE,
                                      FAKE, need, None)
    assert st == _lib.SLAY_E_INVALID  # S is NULL
    st = lib.slay_attn_recurrent_step(ctypes.byref(pd), FAKE, FAKE, FAKE, _lib.SLAY_F32, 10, 64, FAKE, FAKE, FAKE,
                                      FAKE, need - 1, None)
    assert st == _lib.SLAY_E_INVALID and b"workspace too small" in lib.slay_last_error()
    st = lib.slay_attn_recurrent_step(ctypes.byref(pd), FAKE, FAKE, FAKE, _lib.SLAY_F32, 10, 48, FAKE, FAKE, FAKE,
                                      FAKE, need, None)
    assert st == _lib.SLAY_E_UNSUPPORTED and b"decode shape" in lib.slay_last_error()
    st = lib.slay_attn_recurrent_step(ctypes.byref(pd), FAKE, FAKE, FAKE, _lib.SLAY_BF16, 10, 64, FAKE, FAKE, FAKE,
                                      FAKE, need, None)
    assert st == _lib.SLAY_E_UNSUPPORTED  # io dtype must equal the draw dtype
    st = lib.slay_attn_recurrent_step(ctypes.byref(pd), FAKE, FAKE, FAKE, _lib.SLAY_F32, 0, 64, FAKE, FAKE, FAKE,
                                      None, 0, None)
    assert st == _lib.SLAY_OK and lib.slay_last_error() == b""


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def _nc(lib, p, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, dt=_lib.SLAY_BF16, B=1, H=16, Lq=16384, Lk=16384, dv=64, S0=None, z0=None,
                o=FAKE, S_out=None, z_out=None, ws=None, ws_bytes=0)
    args.update(kw)
    return lib.slay_attn_noncausal_fwd(ctypes.byref(p) if p is not None else None, args["q"], args["k"], args["v"],
                                       args["dt"], args["B"], args["H"], args["Lq"], args["Lk"], args["dv"],
                                       args["S0"], args["z0"], args["o"], args["S_out"], args["z_out"], args["ws"],
                                       args["ws_bytes"], None)


def test_noncausal_validation_and_workspace(lib):
    E_INV, E_UNS = _lib.SLAY_E_INVALID, _lib.SLAY_E_UNSUPPORTED
    p = _params()
    assert _nc(lib, None) == E_INV
    assert _nc(lib, p, Lq=-1) == E_INV
    assert _nc(lib, p, Lk=-1) == E_INV
    assert _nc(lib, p, dv=0) == E_INV
    assert _nc(lib, p, dt=_lib.SLAY_F32) == E_UNS
    assert _nc(lib, p, Lk=0) == E_INV and b"no keys" in lib.slay_last_error()
    assert _nc(lib, p, q=None) == E_INV
    assert _nc(lib, p, k=None) == E_INV
    assert _nc(lib, p, o=FAKE + 4) == E_INV
    assert _nc(lib, p) == E_INV and b"workspace too small" in lib.slay_last_error()
    # q and o are not needed without queries, k and v not without keys
    need_k = lib.slay_attn_noncausal_fwd_workspace_size(ctypes.byref(p), 1, 16, 0, 16384, 64, _lib.SLAY_BF16)
    assert _nc(lib, p, q=None, o=None, Lq=0, ws=FAKE, ws_bytes=need_k - 1) == E_INV
    # fused path: 16 key segments per head, their states and the total
    n = lib.slay_attn_noncausal_fwd_workspace_size(ctypes.byref(p), 1, 16, 16384, 16384, 64, _lib.SLAY_BF16)
    assert n == 4 * 16 * 17 * 256 * (64 + 16)
    assert lib.slay_attn_noncausal_fwd_workspace_size(ctypes.byref(p), 1, 16, 100, 0, 64, _lib.SLAY_BF16) == 0
    # general path (fp32): phi(q), phi(k), four 64-key chunk states and their total
    p32 = _params(R=2, m=16, dt=_lib.SLAY_F32)
    n = lib.slay_attn_noncausal_fwd_workspace_size(ctypes.byref(p32), 1, 1, 100, 256, 64, _lib.SLAY_F32)
    assert n == 4 * ((100 + 256) * 32 + 5 * 32 * 65)
    # nothing to do
    assert _nc(lib, p, B=0) == _lib.SLAY_OK


def _bwd(lib, p, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, do=FAKE, dt=_lib.SLAY_BF16, B=1, H=16, L=16384, dv=64, chunk=64, S0=None,
                z0=None, dST=None, dzT=None, dq=FAKE, dk=FAKE, dvo=FAKE, dS0=None, dz0=None, ws=None, ws_bytes=0)
    args.update(kw)
    a = args
    return lib.slay_attn_chunked_bwd(ctypes.byref(p) if p is not None else None, a["q"], a["k"], a["v"], a["do"],
                                     a["dt"], a["B"], a["H"], a["L"], a["dv"], a["chunk"], a["S0"], a["z0"], a["dST"],
                                     a["dzT"], a["dq"], a["dk"], a["dvo"], a["dS0"], a["dz0"], a["ws"], a["ws_bytes"],
                                     None)


def test_backward_validation_and_workspace(lib):
    E_INV, E_UNS = _lib.SLAY_E_INVALID, _lib.SLAY_E_UNSUPPORTED
    p = _params()
    assert _bwd(lib, None) == E_INV
    assert _bwd(lib, p, L=-1) == E_INV
    assert _bwd(lib, p, dv=0) == E_INV
    assert _bwd(lib, p, chunk=0) == E_INV and _bwd(lib, p, chunk=129) == E_INV
    assert _bwd(lib, p, dt=_lib.SLAY_F32) == E_UNS
    assert _bwd(lib, p, dv=512) == E_UNS
    for name in ("q", "k", "v", "do", "dq", "dk", "dvo"):
        assert _bwd(lib, p, **{name: None}) == E_INV, name
        assert _bwd(lib, p, **{name: FAKE + 4}) == E_INV, name
    assert _bwd(lib, p) == E_INV and b"workspace too small" in lib.slay_last_error()
    # MFMA path: one fp32 state per (head, 1024-token segment: about 256 segments in all), an fp32
    # 80-column g' per token and bf16 dphi(q), dphi(k) (phi itself is recomputed on chip)
    n = lib.slay_attn_chunked_bwd_workspace_size(ctypes.byref(p), 1, 16, 16384, 64, 64, _lib.SLAY_BF16)
    rows = 16 * 16384
    assert n == 4 * 16 * 16 * 256 * 80 + 4 * rows * 80 + 2 * 2 * rows * 256
    # general path (fp32): fp32 phi(q), phi(k), dphi(q), dphi(k), g' and one state per chunk
    p32 = _params(R=2, m=16, dt=_lib.SLAY_F32)
    n32 = lib.slay_attn_chunked_bwd_workspace_size(ctypes.byref(p32), 1, 2, 100, 64, 32, _lib.SLAY_F32)
    assert n32 == 4 * (4 * 200 * 32 + 200 * 65 + 2 * 4 * 32 * 65)
    assert _bwd(lib, p, ws=FAKE, ws_bytes=n - 1) == E_INV
    assert _bwd(lib, p, ws=None, ws_bytes=n) == E_INV
    # nothing to do, and no tokens (only the state gradient passes through; no pointers needed)
    assert lib.slay_attn_chunked_bwd_workspace_size(ctypes.byref(p), 1, 16, 0, 64, 64, _lib.SLAY_BF16) == 0
    assert _bwd(lib, p, B=0) == _lib.SLAY_OK


def _vl(lib, p, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dt=_lib.SLAY_BF16, n=4, H=16, cu=FAKE, T=16384, dv=64, S0=None, z0=None,
             o=FAKE, S_out=None, z_out=None, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.slay_attn_varlen_fwd(ctypes.byref(p) if p is not None else None, a["q"], a["k"], a["v"], a["dt"],
                                    a["n"], a["H"], a["cu"], a["T"], a["dv"], a["S0"], a["z0"], a["o"], a["S_out"],
                                    a["z_out"], a["ws"], a["ws_bytes"], None)


def test_varlen_validation_and_workspace(lib):
    E_INV, E_UNS = _lib.SLAY_E_INVALID, _lib.SLAY_E_UNSUPPORTED
    p = _params()
    assert _vl(lib, None) == E_INV
    assert _vl(lib, p, n=-1) == E_INV and _vl(lib, p, H=-1) == E_INV and _vl(lib, p, T=-1) == E_INV
    assert _vl(lib, p, dv=0) == E_INV
    assert _vl(lib, p, dt=_lib.SLAY_F32) == E_UNS
    assert _vl(lib, p, dv=128) == E_UNS and b"variable-length" in lib.slay_last_error()
    assert _vl(lib, _params(R=4, m=16)) == E_UNS  # m must be a multiple of 32
    assert _vl(lib, _params(R=5, m=64)) == E_UNS  # R*m above 256
    assert _vl(lib, p, cu=None) == E_INV
    for name in ("q", "k", "v", "o"):
        assert _vl(lib, p, **{name: None}) == E_INV, name
        assert _vl(lib, p, **{name: FAKE + 4}) == E_INV, name
    assert _vl(lib, p) == E_INV and b"workspace too small" in lib.slay_last_error()
    # one state per (head, state slot), one 16-byte descriptor per work item, the chunk
    # descriptors of the tail packs (at most T / 32 + n_seqs), per-sequence first slot,
    # slot count and last slot, and the item counts of the two passes
    n = lib.slay_attn_varlen_fwd_workspace_size(ctypes.byref(p), 4, 16, 16384, 64, _lib.SLAY_BF16)
    g_max = 16384 // 1024 + 4
    r = lambda b: (b + 255) // 256 * 256
    assert n == r(4 * 16 * g_max * 256 * 80) + r(16 * g_max) + r(16 * (16384 // 32 + 4)) + 3 * r(16) + r(8)
    # more tokens than 2^31 - 65 per head are refused (the work list holds 32-bit token rows)
    assert _vl(lib, p, T=2 ** 31) == E_UNS and b"exceeds" in lib.slay_last_error()
    assert _vl(lib, p, ws=FAKE, ws_bytes=n - 1) == E_INV
    # nothing to do
    assert _vl(lib, p, n=0) == _lib.SLAY_OK and _vl(lib, p, H=0) == _lib.SLAY_OK
    assert lib.slay_attn_varlen_fwd_workspace_size(ctypes.byref(p), 0, 16, 0, 64, _lib.SLAY_BF16) == 0
    # R*m = 96 runs the F = 256 kernels on zero-padded features: the F = 256
    # workspace, then the padded draws (two [1][256][64] bf16) and the padded
    # initial and final states ([4*16][256][64] and [4*16][256] fp32, twice)
    p96 = _params(R=3, m=32)
    n96 = lib.slay_attn_varlen_fwd_workspace_size(ctypes.byref(p96), 4, 16, 16384, 64, _lib.SLAY_BF16)
    assert n96 == r(n) + 2 * r(256 * 64 * 2) + 2 * (r(64 * 256 * 64 * 4) + r(64 * 256 * 4))


def test_noalloc_rejects_before_any_launch(lib):
    """slay_attn_chunked_fwd_noalloc: a workspace beyond the fixed scratch is
    refused on the host (UNSUPPORTED, with the sizes in the message), and bad
    arguments get the same checks as slay_attn_chunked_fwd."""
    E_INV, E_UNS = _lib.SLAY_E_INVALID, _lib.SLAY_E_UNSUPPORTED

    def call(p, B=1, H=8, L=131072, dv=128, chunk=128, q=FAKE):
        return lib.slay_attn_chunked_fwd_noalloc(ctypes.byref(p) if p is not None else None, q, FAKE, FAKE,
                                                 _lib.SLAY_BF16, B, H, L, dv, chunk, None, None, FAKE, None, None,
                                                 None)

    big = _params(d=128, R=4, m=128)
    need = lib.slay_attn_chunked_fwd_workspace_size(ctypes.byref(big), 1, 8, 131072, 128, 128, _lib.SLAY_BF16)
    assert need > _lib.SLAY_NOALLOC_SCRATCH_BYTES
    assert call(big) == E_UNS
    assert b"exceeds the fixed scratch" in lib.slay_last_error()
    assert call(None) == E_INV
    assert call(_params(), H=16, L=16384, dv=64, chunk=0) == E_INV
    assert call(_params(), H=16, L=16384, dv=64, chunk=64, q=None) == E_INV
    # the headline shape's workspace fits the scratch
    fits = lib.slay_attn_chunked_fwd_workspace_size(ctypes.byref(_params()), 1, 16, 16384, 64, 64, _lib.SLAY_BF16)
    assert 0 < fits <= _lib.SLAY_NOALLOC_SCRATCH_BYTES


def test_binding_rejects_mismatched_d_before_launch():
    """Every wrapper compares the last axis of q/k/x with the draws' d before it
    touches the device (a mismatch would make the kernels read or write past
    the tensors)."""
    import types

    import torch

    from kernelized_linear_attention_amd import ops

    fm = types.SimpleNamespace(d=64, F=256, R=4, m=64, n_sets=1)
    x = torch.zeros(2, 3, 5, 48)
    v = torch.zeros(2, 3, 5, 64)
    calls = [
        lambda: ops.featmap(fm, x[0, 0]),
        lambda: ops.chunked_fwd(fm, x, x, v, 64),
        lambda: ops.chunked_fwd_noalloc(fm, x, x, v, 64),
        lambda: ops.chunked_bwd(fm, x, x, v, v, 64),
        lambda: ops.noncausal_fwd(fm, x, x, v),
        lambda: ops.varlen_fwd(fm, x[0], x[0], v[0], torch.zeros(2, dtype=torch.int64)),
        lambda: ops.recurrent_step(fm, x[0, 0], x[0, 0], v[0, 0], torch.zeros(5, 256, 64), torch.zeros(5, 256)),
    ]
    for c in calls:
        with pytest.raises(ValueError, match="d = 64"):
            c()


def test_orthogonal_draws_library(lib):
    """slay_orthogonal_draws: rows orthogonal within blocks of d with the
    lengths of the caller's chi vectors; equal (to fp32 rounding) to the
    sign-fixed QR factor numpy gives for the same Gaussian matrices, and to the
    test inputs' generator fed the same stream."""
    import slay_synth as ss
    from kernelized_linear_attention_amd import ops

    for d, n in ((64, 150), (32, 32), (128, 100)):
        rng = np.random.default_rng([7, d])
        nb = (n + d - 1) // d
        blocks = [(rng.standard_normal((d, d)), rng.standard_normal((d, d))) for _ in range(nb)]
        g = np.stack([b[0] for b in blocks])
        c = np.stack([b[1] for b in blocks])
        out = ops.orthogonal_draws(n, d, g, c).astype(np.float64)
        ref = []
        for b in range(nb):
            Q, R = np.linalg.qr(g[b])
            ref.append((Q * np.sign(np.diag(R))).T * np.linalg.norm(c[b], axis=1)[:, None])
        ref = np.concatenate(ref)[:n]
        np.testing.assert_allclose(out, ref, rtol=0, atol=2e-6 * np.abs(ref).max())
        for b in range(nb):
            blk = out[b * d:(b + 1) * d]
            lens = np.linalg.norm(c[b], axis=1)[:blk.shape[0]]
            np.testing.assert_allclose(np.linalg.norm(blk, axis=1), lens, rtol=1e-6)
            gram = (blk / lens[:, None]) @ (blk / lens[:, None]).T
            np.testing.assert_allclose(gram, np.eye(blk.shape[0]), atol=1e-6)
        synth = ss.orthogonal_gaussian_rows(np.random.default_rng([7, d]), n, d)
        np.testing.assert_allclose(out, synth, rtol=0, atol=2e-6 * np.abs(ref).max())
    a = (ctypes.c_double * 4)()
    f = (ctypes.c_float * 4)()
    assert lib.slay_orthogonal_draws(4, 2, None, a, f) == _lib.SLAY_E_INVALID
    assert lib.slay_orthogonal_draws(4, 0, a, a, f) == _lib.SLAY_E_INVALID
    assert lib.slay_orthogonal_draws(0, 2, None, None, None) == _lib.SLAY_OK
