"""GPU parity of the causal backward through the C ABI against the fp64 oracle.

The backward is the causal forward (review of "SLAY: Geometry-Aware
Spherical Linearized Attention with Yat-Kernel", "Proposed method" bullets
1-6) differentiated; the oracle's backward is pinned to finite differences of
its forward.  Bar as for the forward: 1e-4 for fp32 inputs, 2e-2 for bf16.
Every gradient is gated row by row (helpers.rowfloor_rel): a row's error
relative to its own norm, floored at a tenth of the head's rms row norm.  The
floor is for rows of dq and dk that are legitimately small -- a row of dq is
the projection (I - qh qh^T) of the feature-space gradient, which cancels
where that gradient is nearly parallel to qh -- and for state-gradient rows
of features that carry little weight; a wholly wrong row still fails.
"""
import sys

import numpy as np
import pytest

import slay_synth as ss
from helpers import TOL, headnorm_rel, rowfloor_rel, rownorm_rel, to_dev, to_np

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


def _f32(a):
    import torch

    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _run_bwd(lib, w, q, k, v, dout, A, G, chunk, S0=None, z0=None, dST=None, dzT=None):
    import torch

    fm = lib.FeatureMap(to_dev(A, w.dtype), to_dev(G, w.dtype), w.R, w.m, w.eps)
    res = lib.chunked_bwd(fm, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), to_dev(dout, w.dtype),
                          chunk, S0=_f32(S0), z0=_f32(z0), dS_T=_f32(dST), dz_T=_f32(dzT), state_grad=True)
    torch.cuda.synchronize()
    return tuple(to_np(t) for t in res)


def _state(w, seed):
    rng = np.random.default_rng(seed)
    S0 = np.abs(rng.standard_normal((w.n_heads, w.F, w.dv))).astype(np.float32)
    z0 = (rng.random((w.n_heads, w.F)) + 0.5).astype(np.float32)
    return S0, z0


def _compare(got, ref, dtype, tag):
    dq, dk, dv, dS0, dz0 = got
    rq, rk, rv, rS0, rz0 = ref
    nh = dq.shape[0] * dq.shape[1]
    errs = {
        "dq": rowfloor_rel(dq, rq, heads=nh),
        "dk": rowfloor_rel(dk, rk, heads=nh),
        "dv": rowfloor_rel(dv, rv, heads=nh),
        "dS0": rowfloor_rel(dS0, rS0, heads=nh),
        "dz0": rowfloor_rel(dz0[..., None], rz0[..., None], heads=nh),
    }
    _say(f"  {tag}: " + " ".join(f"{k} {e:.3e}" for k, e in errs.items())
         + f" (unfloored rownorm dq {rownorm_rel(dq, rq):.3e} dk {rownorm_rel(dk, rk):.3e};"
         + f" headnorm dq {headnorm_rel(dq.reshape(nh, -1), rq.reshape(nh, -1)):.3e})")
    for name, e in errs.items():
        assert e < TOL[dtype], (name, e)


@pytest.mark.parametrize("name,B,H,L,chunk,with_state", [
    ("tiny_f32", 1, 2, 100, 32, False),             # fp32, ragged tail
    ("tiny_f32", 1, 2, 77, 16, True),               # fp32 with initial state and final-state gradient
    ("h16_l16k_bf16", 1, 2, 300, 64, True),         # MFMA path: F = 256, three segments, ragged tail
    ("h16_l16k_bf16", 1, 1, 4000, 64, True),        # MFMA path: 32 segments walked in 32-token steps
    ("b4h8_l2k_bf16", 2, 1, 257, 64, False),        # MFMA path on zero-padded features: F = 96, tail of one token
    ("h8_l128k_d128_bf16", 1, 1, 200, 128, True),   # bf16, d = dv = 128, F = 512, chunk 128
])
def test_backward_parity(lib, orc, name, B, H, L, chunk, with_state):
    w = ss.WORKLOADS[name].with_(B=B, H=H, L=L)
    _say(f"backward parity {name} B={B} H={H} L={L} chunk={chunk} state={with_state} dtype={w.dtype}")
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    dout, dST, dzT = ss.make_grads(w)
    S0, z0 = _state(w, 7) if with_state else (None, None)
    if not with_state:
        dST = dzT = None
    got = _run_bwd(lib, w, q, k, v, dout, A, G, chunk, S0, z0, dST, dzT)
    ref = orc.slay_causal_bwd(q, k, v, dout, A, G, w.eps, w.R, w.m, S0=S0, z0=z0, dS_T=dST, dz_T=dzT)
    for t in got:
        assert np.all(np.isfinite(t))
    _compare(got, ref, w.dtype, name)


@pytest.mark.parametrize("R,m,H,L", [
    (3, 32, 2, 700),   # F = 96 (the B4 H8 L2048 workload's features), three segments
    (1, 32, 1, 300),   # F = 32
    (2, 32, 3, 129),   # F = 64
    (7, 32, 1, 1000),  # F = 224
    (8, 32, 2, 400),   # F = 256 itself with eight nodes (no padding)
])
def test_backward_padded_features(lib, orc, R, m, H, L):
    """F < 256 runs the F = 256 MFMA kernels on zero-padded features: the
    padding must change nothing, initial state and final-state gradient included
    (the last case is F = 256 itself, with eight nodes)."""
    w = ss.WORKLOADS["b4h8_l2k_bf16"].with_(B=1, H=H, L=L, R=R, m=m)
    _say(f"backward padded features F={w.F} H={H} L={L}")
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    dout, dST, dzT = ss.make_grads(w)
    S0, z0 = _state(w, 8)
    got = _run_bwd(lib, w, q, k, v, dout, A, G, 64, S0, z0, dST, dzT)
    ref = orc.slay_causal_bwd(q, k, v, dout, A, G, w.eps, w.R, w.m, S0=S0, z0=z0, dS_T=dST, dz_T=dzT)
    for t in got:
        assert np.all(np.isfinite(t))
    assert got[3].shape == (H, w.F, w.dv) and got[4].shape == (H, w.F)
    _compare(got, ref, w.dtype, f"F={w.F}")


def test_backward_padded_per_head_draws(lib, orc):
    """Padded features with one draw set per head (the padding is per set)."""
    import torch

    w = ss.WORKLOADS["b4h8_l2k_bf16"].with_(B=1, H=2, L=256)
    q, k, v = ss.make_qkv(w)
    A0, G0 = ss.make_draws(w)
    A1, G1 = ss.make_draws(w, seed=[3, 98])
    A, G = np.stack([A0, A1]), np.stack([G0, G1])
    dout, _, _ = ss.make_grads(w)
    fm = lib.FeatureMap(to_dev(A, w.dtype), to_dev(G, w.dtype), w.R, w.m, w.eps)
    res = lib.chunked_bwd(fm, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), to_dev(dout, w.dtype), 64,
                          state_grad=True)
    torch.cuda.synchronize()
    got = tuple(to_np(t) for t in res)
    ref = orc.slay_causal_bwd(q, k, v, dout, A, G, w.eps, w.R, w.m, per_head_draws=True)
    _compare(got, ref, w.dtype, "padded, per-head draws")


def test_backward_chunk_invariance(lib):
    """The chunk size changes only the summation order."""
    w = ss.WORKLOADS["tiny_f32"].with_(H=2, L=150)
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    dout, dST, dzT = ss.make_grads(w)
    S0, z0 = _state(w, 9)
    outs = [_run_bwd(lib, w, q, k, v, dout, A, G, c, S0, z0, dST, dzT) for c in (1, 7, 64, 128)]
    for other in outs[1:]:
        for x, y in zip(outs[0], other):
            nh = x.shape[0] * (x.shape[1] if x.ndim == 4 else 1)
            xr = x[..., None] if x.ndim == 2 else x
            yr = y[..., None] if y.ndim == 2 else y
            assert rowfloor_rel(yr, xr, heads=nh) < 1e-5


def test_backward_per_head_draws(lib, orc):
    import torch

    w = ss.WORKLOADS["h16_l16k_bf16"].with_(H=2, L=256)  # whole 128-row tiles per head: the MFMA path
    q, k, v = ss.make_qkv(w)
    A0, G0 = ss.make_draws(w)
    A1, G1 = ss.make_draws(w, seed=[3, 99])
    A, G = np.stack([A0, A1]), np.stack([G0, G1])
    dout, _, _ = ss.make_grads(w)
    fm = lib.FeatureMap(to_dev(A, w.dtype), to_dev(G, w.dtype), w.R, w.m, w.eps)
    res = lib.chunked_bwd(fm, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), to_dev(dout, w.dtype), 64,
                          state_grad=True)
    torch.cuda.synchronize()
    got = tuple(to_np(t) for t in res)
    ref = orc.slay_causal_bwd(q, k, v, dout, A, G, w.eps, w.R, w.m, per_head_draws=True)
    _compare(got, ref, w.dtype, "per-head draws")


def test_backward_split_sequence(lib, orc):
    """Backward through a state handoff: the forward split at token s (second
    part started from the first part's final state) has the same gradients
    as the whole sequence; the second part's dS0 is the first part's dS_T."""
    import torch

    w = ss.WORKLOADS["tiny_f32"].with_(H=2, L=160)
    s = 96
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    dout, _, _ = ss.make_grads(w)
    fm = lib.FeatureMap(to_dev(A, w.dtype), to_dev(G, w.dtype), w.R, w.m, w.eps)
    q_, k_, v_, do_ = (to_dev(x, w.dtype) for x in (q, k, v, dout))
    _, S1, z1 = lib.chunked_fwd(fm, q_[:, :, :s].contiguous(), k_[:, :, :s].contiguous(),
                                v_[:, :, :s].contiguous(), 32, return_state=True)
    part2 = lib.chunked_bwd(fm, q_[:, :, s:].contiguous(), k_[:, :, s:].contiguous(), v_[:, :, s:].contiguous(),
                            do_[:, :, s:].contiguous(), 32, S0=S1, z0=z1, state_grad=True)
    part1 = lib.chunked_bwd(fm, q_[:, :, :s].contiguous(), k_[:, :, :s].contiguous(), v_[:, :, :s].contiguous(),
                            do_[:, :, :s].contiguous(), 32, dS_T=part2[3], dz_T=part2[4], state_grad=True)
    torch.cuda.synchronize()
    got = tuple(np.concatenate([to_np(a), to_np(b)], axis=2) for a, b in zip(part1[:3], part2[:3]))
    got = got + (to_np(part1[3]), to_np(part1[4]))
    ref = orc.slay_causal_bwd(q, k, v, dout, A, G, w.eps, w.R, w.m)
    _compare(got, ref, w.dtype, "split at 96")


def test_backward_edge_cases(lib, orc):
    import torch

    w = ss.WORKLOADS["h16_l16k_bf16"].with_(H=2, L=64)
    A, G = ss.make_draws(w)
    fm = lib.FeatureMap(to_dev(A, w.dtype), to_dev(G, w.dtype), w.R, w.m, w.eps)
    # L = 0: dS0 = dS_T, dz0 = dz_T; without them, zeros
    e = torch.empty(1, 2, 0, w.d, dtype=torch.bfloat16, device="cuda")
    ev = torch.empty(1, 2, 0, w.dv, dtype=torch.bfloat16, device="cuda")
    dST = torch.randn(2, w.F, w.dv, device="cuda")
    dzT = torch.randn(2, w.F, device="cuda")
    dq, dk, dv, dS0, dz0 = lib.chunked_bwd(fm, e, e, ev, ev, 64, dS_T=dST, dz_T=dzT, state_grad=True)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.equal(dS0, dST) and torch.equal(dz0, dzT)
    _, _, _, dS0, dz0 = lib.chunked_bwd(fm, e, e, ev, ev, 64, state_grad=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dS0) == 0 and torch.count_nonzero(dz0) == 0
    # B*H = 0
    e0 = torch.empty(0, 2, 64, w.d, dtype=torch.bfloat16, device="cuda")
    lib.chunked_bwd(fm, e0, e0, e0, e0, 64)
    # one token: o_0 = v_0, so dv_0 = dout_0 and dq_0 = 0
    w1 = w.with_(L=1)
    q, k, v = ss.make_qkv(w1)
    dout, _, _ = ss.make_grads(w1)
    dq, dk, dv, _, _ = _run_bwd(lib, w1, q, k, v, dout, A, G, 64)
    ref = orc.slay_causal_bwd(q, k, v, dout, A, G, w.eps, w.R, w.m)
    assert rownorm_rel(dv, ref[2]) < TOL["bf16"]
    assert np.abs(dq).max() < 1e-2 * np.abs(dout).max() and np.abs(dk).max() < 1e-2 * np.abs(dout).max()


def test_backward_full_size_h16_l16k(lib, orc):
    """The headline shape (B1 H16 L16384, F = 256, chunk 64, bf16) in the
    bench's launch configuration; two whole heads against the oracle."""
    w = ss.WORKLOADS["h16_l16k_bf16"]
    _say("full size h16_l16k_bf16: GPU backward")
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    dout, _, _ = ss.make_grads(w)
    got = _run_bwd(lib, w, q, k, v, dout, A, G, w.chunk)
    for t in got:
        assert np.all(np.isfinite(t))
    for h in (0, 13):
        _say(f"  oracle head {h}")
        sl = slice(h, h + 1)
        ref = orc.slay_causal_bwd(q[:, sl], k[:, sl], v[:, sl], dout[:, sl], A, G, w.eps, w.R, w.m)
        _compare(tuple(x[:, sl] for x in got[:3]) + (got[3][sl], got[4][sl]), ref, w.dtype, f"head {h}")
