"""GPU parity on inputs the workload recipe never produces: q and k rows off
the unit sphere (per-row scales from 1e-3 to 1e3), key rows that are exactly
zero, and query-key pairs with q.k in [0.9, 0.999].

The sphere projection x -> x / max(|x|, 1e-12) is the method's first step
("SLAY: Geometry-Aware Spherical Linearized Attention with Yat-Kernel",
abstract; review, "Proposed method" bullet 1).  The kernels apply it as a
1/|x| scale on the fp32 projection accumulator, and the backward as the
Jacobian (I - xh xh^T)/|x|; on unit-norm inputs both are the identity up to
rounding, so only rows off the sphere test them.  The high-alignment pairs
drive the PRF exponents and the kernel K(u) towards u -> 1, where the
abstract's inverse-square interaction peaks.

Every case runs through the C ABI and is compared with the fp64 oracle on the
same (bf16-rounded where the workload is bf16) values:
  - o, phi: row-normwise relative error (bar 1e-4 fp32, 2e-2 bf16);
  - states and gradients: per-row error floored at a tenth of the head's rms
    row norm (helpers.rowfloor_rel); dq, dk rows are compared after
    multiplying by |q_i|, |k_i|, which removes their 1/|x| scale without
    hiding an error in it (the factor is taken from the inputs, not from
    either result).
A zero key row has phi(k) = 0 (the clamp leaves xh = 0), so it adds nothing
to any state and its gradient is 0; a zero query row would make o = 0/0 and
is not used.  Zero keys are never at token 0 for the same reason.
"""
import sys

import numpy as np
import pytest

import slay_synth as ss
from helpers import TOL, headnorm_rel, rowfloor_rel, rownorm_rel, to_dev, to_np

pytestmark = pytest.mark.gpu

SCALE = (1e-3, 1e3)
NEAR = (0.9, 0.999)


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


def _f32(a):
    import torch

    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _zero_keys(L):
    return [i for i in (1, 2, 63, 64, 65, L // 2, L - 1) if 0 < i < L]


# ----------------------------------------------------------------------------
# feature map

@pytest.mark.parametrize("name,out,rows", [
    ("tiny_f32", "f32", 1000),
    ("h16_l16k_bf16", "bf16", 1000),
    ("h16_l16k_bf16", "f32", 1000),
    ("h16_l16k_bf16", "bf16", 40961),       # large launch: row tiles walked per workgroup
    ("h8_l128k_d128_bf16", "bf16", 1000),
    ("tiny_f32", "f32", 40961),
])
def test_featmap_off_sphere(lib, orc, name, out, rows):
    import torch

    w = ss.WORKLOADS[name].with_(B=1, H=1, L=rows)
    _say(f"featmap off-sphere {name} out={out} rows={rows}")
    _, k, _ = ss.make_qkv(w, qk_scale=SCALE, zero_k=_zero_keys(rows))
    A, G = ss.make_draws(w)
    fm = _fm(lib, w, A, G)
    x = k.reshape(-1, w.d)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    phi = to_np(lib.featmap(fm, to_dev(x, w.dtype), od))
    torch.cuda.synchronize()
    ref = orc.featmap(x, A, G, w.eps, w.R, w.m)
    zero = np.all(x == 0, axis=1)
    err = rownorm_rel(phi[~zero], ref[~zero])
    _say(f"  rownorm rel err {err:.3e}; zero rows {int(zero.sum())}, max |phi| there {np.abs(phi[zero]).max():.1e}")
    assert err < (TOL["bf16"] if out == "bf16" else 1e-4)
    assert np.all(np.isfinite(phi))
    assert np.all(phi[zero] == 0) and np.all(ref[zero] == 0)


@pytest.mark.parametrize("name,out", [("tiny_f32", "f32"), ("h16_l16k_bf16", "bf16"),
                                      ("h8_l128k_d128_bf16", "f32")])
def test_featmap_scale_invariance(lib, name, out):
    """phi(c x) = phi(x) for c > 0: powers of two scale the inputs exactly in
    either dtype, so the GPU's own outputs must agree to rounding."""
    import torch

    w = ss.WORKLOADS[name].with_(B=1, H=1, L=777)
    _, k, _ = ss.make_qkv(w, qk_scale=(0.5, 2.0))
    A, G = ss.make_draws(w)
    fm = _fm(lib, w, A, G)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    base = to_np(lib.featmap(fm, to_dev(k.reshape(-1, w.d), w.dtype), od))
    for c in (2.0 ** -10, 2.0 ** -3, 8.0, 2.0 ** 9):
        got = to_np(lib.featmap(fm, to_dev(k.reshape(-1, w.d) * np.float32(c), w.dtype), od))
        torch.cuda.synchronize()
        err = rownorm_rel(got, base)
        _say(f"  {name} c={c:g}: rel diff {err:.3e}")
        assert err < (1e-2 if out == "bf16" else 1e-5)


# ----------------------------------------------------------------------------
# causal forward on every kernel family

FWD_CASES = [
    # name, overrides, chunk, label
    ("h16_l16k_bf16", dict(H=2, L=2500), 64, "fused F=256"),
    ("b4h8_l2k_bf16", dict(B=1, H=2, L=700), 64, "fused F=96"),
    ("h16_l16k_bf16", dict(H=2, L=700, R=5, m=32), 64, "fused F=160 padded"),
    ("h8_l128k_d128_bf16", dict(H=2, L=1000), 128, "wide d=128 F=512"),
    ("h16_l16k_bf16", dict(H=2, L=700), 32, "wide d=64 F=256"),
    ("b4h8_l2k_bf16", dict(B=1, H=2, L=500), 32, "general bf16"),
    ("tiny_f32", dict(H=2, L=300), 32, "general fp32"),
]


@pytest.mark.parametrize("name,over,chunk,label", FWD_CASES)
@pytest.mark.parametrize("stress", ["scaled", "near", "near_scaled"])
def test_causal_stress_inputs(lib, orc, name, over, chunk, label, stress):
    w = ss.WORKLOADS[name].with_(**over, chunk=chunk)
    _say(f"causal {stress} {label}: B={w.B} H={w.H} L={w.L} F={w.F} chunk={chunk}")
    kw = {}
    if "scaled" in stress:
        kw.update(qk_scale=SCALE, zero_k=_zero_keys(w.L))
    if "near" in stress:
        kw.update(near_pairs=NEAR)
    q, k, v = ss.make_qkv(w, **kw)
    A, G = ss.make_draws(w)
    fm = _fm(lib, w, A, G)
    import torch

    o, S, z = lib.chunked_fwd(fm, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), chunk,
                              return_state=True)
    torch.cuda.synchronize()
    o, S, z = to_np(o), to_np(S), to_np(z)
    ro, rS, rz = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m, form="recurrent")
    nh = w.B * w.H
    err = rownorm_rel(o, ro)
    s_err = rowfloor_rel(S, rS, heads=nh)
    z_err = rowfloor_rel(z[..., None], rz[..., None], heads=nh)
    _say(f"  o rownorm {err:.3e}; S per-row {s_err:.3e} (headnorm {headnorm_rel(S, rS):.3e}); z per-row {z_err:.3e}")
    tol = TOL[w.dtype]
    assert np.all(np.isfinite(o))
    assert err < tol and s_err < tol and z_err < tol


@pytest.mark.parametrize("R,m,d,chunk,label", [
    (16, 16, 64, 64, "R=16 wide"),
    (16, 16, 64, 16, "R=16 general"),
    (8, 32, 64, 64, "R=8 fused"),
])
def test_causal_near_pairs_many_nodes(lib, orc, R, m, d, chunk, label):
    """The high-alignment set with the most Gauss-Laguerre nodes (largest beta_r)."""
    import torch

    w = ss.WORKLOADS["h16_l16k_bf16"].with_(H=2, L=600, R=R, m=m, d=d, chunk=chunk)
    _say(f"near pairs {label}: F={w.F}")
    q, k, v = ss.make_qkv(w, near_pairs=NEAR, qk_scale=(0.1, 10.0))
    A, G = ss.make_draws(w)
    fm = _fm(lib, w, A, G)
    o, S, z = lib.chunked_fwd(fm, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), chunk,
                              return_state=True)
    torch.cuda.synchronize()
    ro, rS, rz = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m)
    err = rownorm_rel(to_np(o), ro)
    s_err = rowfloor_rel(to_np(S), rS, heads=2)
    _say(f"  o rownorm {err:.3e}; S per-row {s_err:.3e}")
    assert err < TOL["bf16"] and s_err < TOL["bf16"]


def test_causal_full_size_off_sphere(lib, orc):
    """The headline launch (B1 H16 L16384, F=256, chunk 64) with scaled rows,
    zero keys and high-alignment pairs; sampled rows of two heads are summed
    one by one by the oracle."""
    import torch

    w = ss.WORKLOADS["h16_l16k_bf16"]
    _say("full size h16_l16k_bf16 off-sphere: GPU forward")
    q, k, v = ss.make_qkv(w, qk_scale=SCALE, near_pairs=NEAR, zero_k=_zero_keys(w.L))
    A, G = ss.make_draws(w)
    fm = _fm(lib, w, A, G)
    o = to_np(lib.chunked_fwd(fm, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), w.chunk))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(o))
    rows = np.array([0, 1, 2, 63, 64, 1023, 1024, 1025, 8191, 12345, w.L - 1])
    for h in (0, 9):
        phk = orc.featmap(k[0, h], A, G, w.eps, w.R, w.m)
        phq = orc.featmap(q[0, h, rows], A, G, w.eps, w.R, w.m)
        ref = orc.attn_rows(rows, phq, phk, v[0, h])
        err = rownorm_rel(o[0, h, rows], ref)
        _say(f"  head {h}: sampled rows rownorm {err:.3e}")
        assert err < TOL["bf16"]


# ----------------------------------------------------------------------------
# non-causal, variable-length, decode

@pytest.mark.parametrize("name,H,Lq,Lk", [
    ("h16_l16k_bf16", 2, 700, 3000),       # fused, several key segments
    ("b4h8_l2k_bf16", 2, 300, 500),        # fused F = 96
    ("h8_l128k_d128_bf16", 1, 300, 500),   # general bf16
    ("tiny_f32", 2, 200, 300),             # general fp32
])
def test_noncausal_stress_inputs(lib, orc, name, H, Lq, Lk):
    import torch

    w = ss.WORKLOADS[name].with_(B=1, H=H, L=max(Lq, Lk))
    _say(f"noncausal off-sphere {name} H={H} Lq={Lq} Lk={Lk}")
    q, k, v = ss.make_qkv(w, qk_scale=SCALE, near_pairs=NEAR, zero_k=_zero_keys(Lk))
    q, k, v = q[:, :, :Lq], k[:, :, :Lk], v[:, :, :Lk]
    A, G = ss.make_draws(w)
    fm = _fm(lib, w, A, G)
    o, S, z = lib.noncausal_fwd(fm, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype),
                                return_state=True)
    torch.cuda.synchronize()
    ro, rS, rz = orc.slay_noncausal(q, k, v, A, G, w.eps, w.R, w.m)
    err = rownorm_rel(to_np(o), ro)
    s_err = rowfloor_rel(to_np(S), rS, heads=H)
    z_err = rowfloor_rel(to_np(z)[..., None], rz[..., None], heads=H)
    _say(f"  o rownorm {err:.3e}; S per-row {s_err:.3e}; z per-row {z_err:.3e}")
    tol = TOL[w.dtype]
    assert err < tol and s_err < tol and z_err < tol


def test_varlen_stress_inputs(lib, orc):
    import torch

    W = ss.WORKLOADS["h16_l16k_bf16"]
    H, lengths = 2, [300, 1, 1000, 77, 2049]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1])
    zk = [int(cu[s]) + 5 for s in range(len(lengths)) if lengths[s] > 5]
    q, k, v = ss.make_qkv(W.with_(B=1, H=H, L=T), seed=[3, 75], qk_scale=SCALE, near_pairs=NEAR, zero_k=zk)
    q, k, v = q[0], k[0], v[0]
    A, G = ss.make_draws(W)
    fm = _fm(lib, W, A, G)
    o, S, z = lib.varlen_fwd(fm, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                             torch.from_numpy(cu).cuda(), return_state=True)
    torch.cuda.synchronize()
    ro, rS, rz = orc.slay_causal_varlen(q, k, v, cu, A, G, W.eps, W.R, W.m)
    n = len(lengths) * H
    err = rownorm_rel(to_np(o), ro)
    s_err = rowfloor_rel(to_np(S).reshape(n, W.F, W.dv), rS.reshape(n, W.F, W.dv), heads=n)
    z_err = rowfloor_rel(to_np(z).reshape(n, W.F, 1), rz.reshape(n, W.F, 1), heads=n)
    _say(f"varlen off-sphere: o rownorm {err:.3e}; S per-row {s_err:.3e}; z per-row {z_err:.3e}")
    assert err < TOL["bf16"] and s_err < TOL["bf16"] and z_err < TOL["bf16"]


def test_decode_stress_inputs(lib, orc):
    """fp32 decode steps with scaled q, k rows and zero keys at later steps."""
    import torch

    w = ss.WORKLOADS["decode_256x16_f32"]
    n_heads, steps = 64, 200
    A, G = ss.make_draws(w)
    qs, ks, vs = [], [], []
    for t in range(steps):
        q, k, v = ss.make_decode_step(w, t, n_heads, qk_scale=SCALE)
        if t in (1, 7, 150):
            k = k.copy()
            k[::3] = 0.0
        qs.append(q)
        ks.append(k)
        vs.append(v)
    q, k, v = np.stack(qs, 1), np.stack(ks, 1), np.stack(vs, 1)
    fm = _fm(lib, w, A, G)
    S = torch.zeros(n_heads, w.F, w.dv, device="cuda")
    z = torch.zeros(n_heads, w.F, device="cuda")
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    outs = torch.empty(n_heads, steps, w.dv, device="cuda")
    for t in range(steps):
        outs[:, t] = lib.recurrent_step(fm, qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(), S, z)
    torch.cuda.synchronize()
    ro, rS, rz = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m, form="recurrent")
    err = rownorm_rel(to_np(outs), ro)
    s_err = rowfloor_rel(to_np(S), rS, heads=n_heads)
    z_err = rowfloor_rel(to_np(z)[..., None], rz[..., None], heads=n_heads)
    _say(f"decode off-sphere: o rownorm {err:.3e}; S per-row {s_err:.3e}; z per-row {z_err:.3e}")
    assert err < TOL["f32"] and s_err < TOL["f32"] and z_err < TOL["f32"]
# ----------------------------------------------------------------------------
# backward: the sphere projection's Jacobian (I - xh xh^T)/|x| and the clamp

BWD_CASES = [
    ("h16_l16k_bf16", dict(H=2, L=1500), 64, "MFMA F=256"),
    ("b4h8_l2k_bf16", dict(B=1, H=2, L=700), 64, "MFMA F=96 padded"),
    ("h8_l128k_d128_bf16", dict(H=1, L=300), 128, "general bf16 d=128"),
    ("tiny_f32", dict(H=2, L=200), 32, "general fp32"),
]


@pytest.mark.parametrize("name,over,chunk,label", BWD_CASES)
@pytest.mark.parametrize("stress", ["scaled", "near_scaled"])
def test_backward_stress_inputs(lib, orc, name, over, chunk, label, stress):
    import torch

    w = ss.WORKLOADS[name].with_(**over)
    _say(f"backward {stress} {label}: H={w.H} L={w.L} F={w.F}")
    kw = dict(qk_scale=SCALE, zero_k=_zero_keys(w.L))
    if stress == "near_scaled":
        kw.update(near_pairs=NEAR)
    q, k, v = ss.make_qkv(w, **kw)
    A, G = ss.make_draws(w)
    dout, dST, dzT = ss.make_grads(w)
    rng = np.random.default_rng(17)
    S0 = np.abs(rng.standard_normal((w.n_heads, w.F, w.dv))).astype(np.float32)
    z0 = (rng.random((w.n_heads, w.F)) + 0.5).astype(np.float32)
    fm = _fm(lib, w, A, G)
    res = lib.chunked_bwd(fm, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), to_dev(dout, w.dtype),
                          chunk, S0=_f32(S0), z0=_f32(z0), dS_T=_f32(dST), dz_T=_f32(dzT), state_grad=True)
    torch.cuda.synchronize()
    dq, dk, dv, dS0, dz0 = (to_np(t) for t in res)
    rq, rk, rv, rS0, rz0 = orc.slay_causal_bwd(q, k, v, dout, A, G, w.eps, w.R, w.m, S0=S0, z0=z0, dS_T=dST,
                                                dz_T=dzT)
    nh = w.n_heads
    nq = np.linalg.norm(q.astype(np.float64), axis=-1, keepdims=True)
    nk = np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True)
    zero = nk[..., 0] == 0
    errs = {
        "dq": rowfloor_rel(nq * dq, nq * rq, heads=nh),
        "dk": rowfloor_rel(nk * dk, nk * rk, heads=nh),
        "dv": rowfloor_rel(dv, rv, heads=nh),
        "dS0": rowfloor_rel(dS0, rS0, heads=nh),
        "dz0": rowfloor_rel(dz0[..., None], rz0[..., None], heads=nh),
    }
    _say("  " + " ".join(f"{n} {e:.3e}" for n, e in errs.items())
         + f"; dk on zero keys max {np.abs(dk[zero]).max() if zero.any() else 0:.1e}")
    for t in (dq, dk, dv, dS0, dz0):
        assert np.all(np.isfinite(t))
    assert np.all(rk[zero] == 0) and np.all(dk[zero] == 0)
    for n, e in errs.items():
        assert e < TOL[w.dtype], (n, e)
