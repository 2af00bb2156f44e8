"""GPU parity of the non-causal forward (every query attends to every key)
through the C ABI against the fp64 oracle.

Method: the standard linear-attention contraction over all keys (review of
"SLAY: Geometry-Aware Spherical Linearized Attention with Yat-Kernel",
"Proposed method" bullet 6).  Bar as for the causal forward: row-normwise
1e-4 for fp32 inputs, 2e-2 for bf16; the final state row by row, floored
at a tenth of the head's rms row norm (helpers.rowfloor_rel).
"""
import sys

import numpy as np
import pytest

import slay_synth as ss
from helpers import TOL, elem_rel, headnorm_rel, rowfloor_rel, rownorm_rel, to_dev, to_np

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


def _fm(ops, w, A, G):
    return ops.FeatureMap(to_dev(A, w.dtype), to_dev(G, w.dtype), w.R, w.m, w.eps)


def _srel(S, rS):
    """States [heads, F, dv]: per-row error, floored per head."""
    return rowfloor_rel(S, rS, heads=S.shape[0])


def _zrel(z, rz):
    """z [heads, F]: per-feature error, floored per head."""
    return rowfloor_rel(z[..., None], rz[..., None], heads=z.shape[0])


def _inputs(w, Lq, Lk):
    """Queries from the workload's q stream, keys/values from its k/v streams."""
    q, k, v = ss.make_qkv(w.with_(L=max(Lq, Lk)))
    return q[:, :, :Lq], k[:, :, :Lk], v[:, :, :Lk]


def _run(lib, w, q, k, v, A, G, S0=None, z0=None, state=False):
    import torch

    fm = _fm(lib, w, A, G)
    S0d = None if S0 is None else torch.from_numpy(np.float32(S0)).cuda()
    z0d = None if z0 is None else torch.from_numpy(np.float32(z0)).cuda()
    res = lib.noncausal_fwd(fm, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), S0=S0d, z0=z0d,
                            return_state=state)
    torch.cuda.synchronize()
    if state:
        return tuple(to_np(t) for t in res)
    return to_np(res)


@pytest.mark.parametrize("name,B,H,Lq,Lk", [
    ("tiny_f32", 1, 2, 200, 300),            # general path, fp32
    ("b4h8_l2k_bf16", 1, 2, 500, 700),       # fused, F = 96 (6 feature waves)
    ("h16_l16k_bf16", 1, 3, 700, 1000),      # fused, F = 256, ragged chunks, one key segment
    ("h16_l16k_bf16", 1, 2, 64, 5000),       # fused, several key segments
    ("h8_l128k_d128_bf16", 1, 2, 300, 500),  # general path, bf16, d = 128, F = 512
])
def test_noncausal_parity(lib, orc, name, B, H, Lq, Lk):
    w = ss.WORKLOADS[name].with_(B=B, H=H)
    _say(f"noncausal parity {name} B={B} H={H} Lq={Lq} Lk={Lk} dtype={w.dtype}")
    q, k, v = _inputs(w, Lq, Lk)
    A, G = ss.make_draws(w)
    o, S, z = _run(lib, w, q, k, v, A, G, state=True)
    ro, rS, rz = orc.slay_noncausal(q, k, v, A, G, w.eps, w.R, w.m)
    err = rownorm_rel(o, ro)
    s_err, z_err = _srel(S, rS), _zrel(z, rz)
    _say(f"  o rownorm rel err {err:.3e} elementwise {elem_rel(o, ro):.3e}; S {s_err:.3e} z {z_err:.3e}"
         f" (headnorm S {headnorm_rel(S, rS):.3e})")
    assert err < TOL[w.dtype]
    assert s_err < TOL[w.dtype] and z_err < TOL[w.dtype]


def test_noncausal_initial_state_and_split(lib, orc):
    """Keys in two calls with the state carried equal one call; S_out may alias S0."""
    import torch

    for name in ("tiny_f32", "h16_l16k_bf16"):
        w = ss.WORKLOADS[name].with_(H=2)
        Lq, Lk, cut = 300, 900, 400
        _say(f"noncausal state split {name}")
        q, k, v = _inputs(w, Lq, Lk)
        A, G = ss.make_draws(w)
        _, S1, z1 = _run(lib, w, q, k[:, :, :cut], v[:, :, :cut], A, G, state=True)
        o2, S2, z2 = _run(lib, w, q, k[:, :, cut:], v[:, :, cut:], A, G, S0=S1, z0=z1, state=True)
        ro, rS, rz = orc.slay_noncausal(q, k, v, A, G, w.eps, w.R, w.m)
        assert rownorm_rel(o2, ro) < TOL[w.dtype]
        assert _srel(S2, rS) < TOL[w.dtype] and _zrel(z2, rz) < TOL[w.dtype]
        # in place: S_out aliases S0
        fm = _fm(lib, w, A, G)
        S = torch.from_numpy(np.float32(S1)).cuda()
        z = torch.from_numpy(np.float32(z1)).cuda()
        o3 = lib.noncausal_fwd(fm, to_dev(q, w.dtype), to_dev(k[:, :, cut:], w.dtype), to_dev(v[:, :, cut:], w.dtype),
                               S0=S, z0=z, S_out=S, z_out=z, return_state=True)[0]
        torch.cuda.synchronize()
        assert rownorm_rel(to_np(o3), ro) < TOL[w.dtype]
        assert _srel(to_np(S), rS) < TOL[w.dtype]


@pytest.mark.parametrize("R,m,per_head", [(5, 16, False), (7, 32, True), (4, 16, False), (2, 64, True)])
def test_noncausal_padded_features(lib, orc, R, m, per_head):
    """F = 80 and F = 224 on zero-padded features, F = 64 and F = 128 on their own kernels, with an
    initial state and the final state out."""
    w = ss.WORKLOADS["h16_l16k_bf16"].with_(B=1, H=2, R=R, m=m)
    _say(f"noncausal padded F={w.F} per_head={per_head}")
    q, k, v = _inputs(w, 300, 900)
    if per_head:
        draws = [ss.make_draws(w, seed=[3, 60 + h]) for h in range(w.H)]
        A, G = np.stack([a for a, _ in draws]), np.stack([g for _, g in draws])
    else:
        A, G = ss.make_draws(w)
    rng = np.random.default_rng(12)
    S0 = np.abs(rng.standard_normal((w.H, w.F, w.dv))).astype(np.float32)
    z0 = (rng.random((w.H, w.F)) + 0.5).astype(np.float32)
    o, S, z = _run(lib, w, q, k, v, A, G, S0=S0, z0=z0, state=True)
    ro, rS, rz = orc.slay_noncausal(q, k, v, A, G, w.eps, w.R, w.m, S0=S0, z0=z0, per_head_draws=per_head)
    err = rownorm_rel(o, ro)
    s_err = _srel(S.reshape(w.H, w.F, -1), rS.reshape(w.H, w.F, -1))
    z_err = _zrel(z.reshape(w.H, -1), rz.reshape(w.H, -1))
    _say(f"  o rownorm {err:.3e}; S {s_err:.3e} z {z_err:.3e}")
    assert S.shape == (w.H, w.F, w.dv)
    assert err < TOL["bf16"] and s_err < TOL["bf16"] and z_err < TOL["bf16"]


def test_noncausal_edge_cases(lib, orc):
    import torch
    from kernelized_linear_attention_amd import _lib

    # the last case runs F = 80 on zero-padded features
    for name, extra in (("tiny_f32", {}), ("h16_l16k_bf16", {}), ("h16_l16k_bf16", {"R": 5, "m": 16})):
        w = ss.WORKLOADS[name].with_(H=2, **extra)
        _say(f"noncausal edge cases {name} F={w.F}")
        q, k, v = _inputs(w, 130, 200)
        A, G = ss.make_draws(w)
        _, S1, z1 = orc.slay_noncausal(q, k, v, A, G, w.eps, w.R, w.m)
        # no keys: the output is the readout of the initial state
        o0, S0o, z0o = _run(lib, w, q, k[:, :, :0], v[:, :, :0], A, G, S0=S1, z0=z1, state=True)
        ro = orc.slay_noncausal(q, k[:, :, :0], v[:, :, :0], A, G, w.eps, w.R, w.m, S0=S1, z0=z1)[0]
        assert rownorm_rel(o0, ro) < TOL[w.dtype]
        np.testing.assert_allclose(S0o, np.float32(S1), rtol=0, atol=0)
        # no queries: only the state
        oq, Sq, zq = _run(lib, w, q[:, :, :0], k, v, A, G, state=True)
        assert oq.size == 0 and _srel(Sq, S1) < TOL[w.dtype] and _zrel(zq, z1) < TOL[w.dtype]
        # no keys and no initial state: rejected before any launch
        fm = _fm(lib, w, A, G)
        with pytest.raises(_lib.SlayError, match="no keys"):
            lib.noncausal_fwd(fm, to_dev(q, w.dtype), to_dev(k[:, :, :0], w.dtype), to_dev(v[:, :, :0], w.dtype))
        # B*H = 0
        e0 = torch.empty(0, 2, 64, w.d, dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32, device="cuda")
        lib.noncausal_fwd(fm, e0, e0, torch.empty(0, 2, 64, w.dv, dtype=e0.dtype, device="cuda"))


def test_noncausal_full_size_h16_l16k_sampled(lib, orc):
    """Headline shape (B1 H16, Lq = Lk = 16384, bf16, F = 256) in the bench's launch
    configuration; each query's output depends only on it and all keys, so sampled
    queries of two heads are checked exactly, and those heads' final states."""
    w = ss.WORKLOADS["h16_l16k_bf16"]
    _say("noncausal full size h16_l16k_bf16: GPU forward")
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    o, S, z = _run(lib, w, q, k, v, A, G, state=True)
    assert np.all(np.isfinite(o))
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(w.L, 48, replace=False))
    for h in (0, 13):
        _say(f"  oracle head {h}")
        ro, rS, rz = orc.slay_noncausal(q[:, h:h + 1, rows], k[:, h:h + 1], v[:, h:h + 1], A, G, w.eps, w.R, w.m)
        err = rownorm_rel(o[:, h:h + 1, rows], ro)
        s_err = _srel(S[h:h + 1], rS)
        _say(f"  head {h}: o rownorm rel err {err:.3e}; S {s_err:.3e}")
        assert err < TOL["bf16"] and s_err < TOL["bf16"]
    # every output inside the hull of its head's values
    lo = v.min(axis=2, keepdims=True)
    hi = v.max(axis=2, keepdims=True)
    slack = 0.02 * (hi - lo)
    assert np.all(o >= lo - slack) and np.all(o <= hi + slack)
