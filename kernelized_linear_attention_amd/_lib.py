"""ctypes view of the C ABI declared in include/slay.h (marshalling only)."""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libslay.so")

SLAY_OK, SLAY_E_INVALID, SLAY_E_UNSUPPORTED, SLAY_E_DEVICE = 0, 1, 2, 3
SLAY_F32, SLAY_BF16 = 0, 1
SLAY_NOALLOC_SCRATCH_BYTES = 32 << 20  # include/slay.h

# every function include/slay.h declares
EXPORTS = ("slay_featmap", "slay_attn_chunked_fwd_workspace_size", "slay_attn_chunked_fwd", "slay_attn_chunked_fwd_noalloc",
           "slay_attn_varlen_fwd_workspace_size", "slay_attn_varlen_fwd",
           "slay_attn_chunked_bwd_workspace_size", "slay_attn_chunked_bwd",
           "slay_attn_noncausal_fwd_workspace_size", "slay_attn_noncausal_fwd",
           "slay_attn_recurrent_step_workspace_size", "slay_attn_recurrent_step", "slay_gl_table", "slay_orthogonal_draws",
           "slay_status_string", "slay_last_error", "slay_version")


class SlayParams(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("R", ctypes.c_int32), ("m", ctypes.c_int32), ("eps", ctypes.c_double),
                ("anchors", ctypes.c_void_p), ("prf", ctypes.c_void_p), ("draw_dtype", ctypes.c_int),
                ("n_draw_sets", ctypes.c_int32), ("draw_set_stride", ctypes.c_int64)]


class SlayError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """Load libslay.so; raises if it has not been built (there is no fallback).

    PyTorch-ROCm ships its own HIP runtime.  One process must hold a single
    HIP runtime, so torch (when installed) is imported first and libslay's
    libamdhip64 dependency resolves to the runtime torch already loaded.
    """
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m kernelized_linear_attention_amd.build`")
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(SlayParams)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        fp = ctypes.c_void_p
        lib.slay_featmap.argtypes = [P, vp, ctypes.c_int, i64, i64, vp, ctypes.c_int, vp]
        lib.slay_featmap.restype = ctypes.c_int
        lib.slay_attn_chunked_fwd_workspace_size.argtypes = [P, i32, i32, i64, i32, i32, ctypes.c_int]
        lib.slay_attn_chunked_fwd_workspace_size.restype = sz
        lib.slay_attn_chunked_fwd.argtypes = [P, vp, vp, vp, ctypes.c_int, i32, i32, i64, i32, i32, fp, fp, vp, fp,
                                              fp, vp, sz, vp]
        lib.slay_attn_chunked_fwd.restype = ctypes.c_int
        lib.slay_attn_chunked_fwd_noalloc.argtypes = [P, vp, vp, vp, ctypes.c_int, i32, i32, i64, i32, i32, fp, fp,
                                                      vp, fp, fp, vp]
        lib.slay_attn_chunked_fwd_noalloc.restype = ctypes.c_int
        lib.slay_attn_varlen_fwd_workspace_size.argtypes = [P, i32, i32, i64, i32, ctypes.c_int]
        lib.slay_attn_varlen_fwd_workspace_size.restype = sz
        lib.slay_attn_varlen_fwd.argtypes = [P, vp, vp, vp, ctypes.c_int, i32, i32, vp, i64, i32, fp, fp, vp, fp, fp,
                                             vp, sz, vp]
        lib.slay_attn_varlen_fwd.restype = ctypes.c_int
        lib.slay_attn_chunked_bwd_workspace_size.argtypes = [P, i32, i32, i64, i32, i32, ctypes.c_int]
        lib.slay_attn_chunked_bwd_workspace_size.restype = sz
        lib.slay_attn_chunked_bwd.argtypes = [P, vp, vp, vp, vp, ctypes.c_int, i32, i32, i64, i32, i32, fp, fp, fp,
                                              fp, vp, vp, vp, fp, fp, vp, sz, vp]
        lib.slay_attn_chunked_bwd.restype = ctypes.c_int
        lib.slay_attn_noncausal_fwd_workspace_size.argtypes = [P, i32, i32, i64, i64, i32, ctypes.c_int]
        lib.slay_attn_noncausal_fwd_workspace_size.restype = sz
        lib.slay_attn_noncausal_fwd.argtypes = [P, vp, vp, vp, ctypes.c_int, i32, i32, i64, i64, i32, fp, fp, vp,
                                                fp, fp, vp, sz, vp]
        lib.slay_attn_noncausal_fwd.restype = ctypes.c_int
        lib.slay_attn_recurrent_step_workspace_size.argtypes = [P, i64, i32, ctypes.c_int]
        lib.slay_attn_recurrent_step_workspace_size.restype = sz
        lib.slay_attn_recurrent_step.argtypes = [P, vp, vp, vp, ctypes.c_int, i64, i32, fp, fp, vp, vp, sz, vp]
        lib.slay_attn_recurrent_step.restype = ctypes.c_int
        lib.slay_gl_table.argtypes = [i32, ctypes.c_double, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_double)]
        lib.slay_gl_table.restype = ctypes.c_int
        dp = ctypes.POINTER(ctypes.c_double)
        lib.slay_orthogonal_draws.argtypes = [i32, i32, dp, dp, ctypes.POINTER(ctypes.c_float)]
        lib.slay_orthogonal_draws.restype = ctypes.c_int
        lib.slay_status_string.argtypes = [ctypes.c_int]
        lib.slay_status_string.restype = ctypes.c_char_p
        lib.slay_last_error.argtypes = []
        lib.slay_last_error.restype = ctypes.c_char_p
        lib.slay_version.argtypes = []
        lib.slay_version.restype = ctypes.c_int32
        _lib = lib
        return lib


def check(status: int, what: str) -> None:
    if status != SLAY_OK:
        lib = load()
        msg = lib.slay_last_error().decode() or lib.slay_status_string(status).decode()
        raise SlayError(status, f"{what}: {msg}")
