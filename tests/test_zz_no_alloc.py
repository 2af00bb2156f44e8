"""slay_attn_chunked_fwd_noalloc (the forward for callers that cannot allocate)
against slay_attn_chunked_fwd, both through the C ABI.

The no-allocation entry point runs the same kernels with the library's fixed
device scratch in place of the caller's workspace, so on the same inputs its
outputs and final states must equal the workspace entry point's exactly.  Two
calls in a row, the second on a smaller problem, check that nothing the first
call left in the shared scratch leaks into the second.  The bar otherwise is
the parity bar of the forward (row-normwise 2e-2 for bf16, 1e-4 for fp32).
"""
import sys

import numpy as np
import pytest

import slay_synth as ss
from helpers import TOL, rownorm_rel, to_dev, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from kernelized_linear_attention_amd import ops

    return ops


def _case(lib, w, seed, with_state):
    import torch

    q, k, v = (to_dev(a, w.dtype) for a in ss.make_qkv(w, seed=seed))
    A, G = ss.make_draws(w)
    fm = lib.FeatureMap(to_dev(A, w.dtype), to_dev(G, w.dtype), w.R, w.m, w.eps)
    S0 = z0 = None
    if with_state:
        rng = np.random.default_rng(seed + [1])
        S0 = torch.from_numpy(np.abs(rng.standard_normal((w.n_heads, w.F, w.dv))).astype(np.float32)).cuda()
        z0 = torch.from_numpy((rng.random((w.n_heads, w.F)) + 0.5).astype(np.float32)).cuda()
    ref = lib.chunked_fwd(fm, q, k, v, w.chunk, S0=S0, z0=z0, return_state=True)
    got = lib.chunked_fwd_noalloc(fm, q, k, v, w.chunk, S0=S0, z0=z0, return_state=True)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("first,second", [
    # the headline launch (F = 256 fused kernels, 16 segments per head), then a smaller ragged one
    (dict(name="h16_l16k_bf16", over={}, state=False), dict(name="h16_l16k_bf16", over=dict(H=3, L=1000), state=True)),
    # zero-padded features (F = 96 -> built F = 96, B4 H8 L2048), then F = 160 on the F = 256 kernels
    (dict(name="b4h8_l2k_bf16", over={}, state=True), dict(name="h16_l16k_bf16", over=dict(H=2, L=700, R=5, m=32),
                                                          state=False)),
    # the general fp32 path (its workspace: phi and per-chunk states), twice
    (dict(name="tiny_f32", over=dict(H=4), state=True), dict(name="tiny_f32", over=dict(L=200), state=False)),
])
def test_noalloc_matches_workspace_entry_point(lib, orc, first, second):
    import torch

    for i, c in enumerate((first, second)):
        w = ss.WORKLOADS[c["name"]].with_(**c["over"])
        _say(f"noalloc call {i}: {c['name']} B={w.B} H={w.H} L={w.L} F={w.F} state={c['state']}")
        (o_r, S_r, z_r), (o_g, S_g, z_g) = _case(lib, w, [w.wid, 40 + i], c["state"])
        err = rownorm_rel(to_np(o_g), to_np(o_r))
        same = torch.equal(o_g, o_r) and torch.equal(S_g, S_r) and torch.equal(z_g, z_r)
        _say(f"  vs workspace entry point: o rownorm {err:.3e}, bit-identical {same}")
        assert err < TOL[w.dtype]
        assert rownorm_rel(to_np(S_g).reshape(-1, w.dv), to_np(S_r).reshape(-1, w.dv)) < TOL[w.dtype]
        assert same
        if w.L * w.n_heads <= 4 * 1024:
            q, k, v = ss.make_qkv(w, seed=[w.wid, 40 + i])
            A, G = ss.make_draws(w)
            S0 = z0 = None
            if c["state"]:
                rng = np.random.default_rng([w.wid, 40 + i, 1])
                S0 = np.abs(rng.standard_normal((w.n_heads, w.F, w.dv))).astype(np.float32)
                z0 = (rng.random((w.n_heads, w.F)) + 0.5).astype(np.float32)
            ro = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m, S0=S0, z0=z0)[0]
            assert rownorm_rel(to_np(o_g), ro) < TOL[w.dtype]


def test_noalloc_refuses_oversized_workspace(lib):
    """A shape whose workspace exceeds the fixed scratch is refused before anything is enqueued."""
    import torch

    from kernelized_linear_attention_amd import _lib

    w = ss.WORKLOADS["h8_l128k_d128_bf16"]
    fm = lib.FeatureMap(torch.zeros(w.F, w.d, dtype=torch.bfloat16, device="cuda"),
                        torch.zeros(w.F, w.d, dtype=torch.bfloat16, device="cuda"), w.R, w.m, w.eps)
    x = torch.zeros(1, 8, w.L, w.d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.SlayError, match="exceeds the fixed scratch"):
        lib.chunked_fwd_noalloc(fm, x, x, x, w.chunk)
    torch.cuda.synchronize()
