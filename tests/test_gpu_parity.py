"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Both sides read the same seeded inputs and the same anchor / PRF draws
(bf16 workloads: the bf16-rounded values, upcast exactly for the oracle).
Bar: row-normwise max relative error 1e-4 for fp32 inputs, 2e-2 for bf16.
"""
import sys

import numpy as np
import pytest

import slay_synth as ss
from helpers import TOL, elem_rel, headnorm_rel, rowfloor_rel, rownorm_rel, to_dev, to_np, torch_dtype

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


# ----------------------------------------------------------------------------
# feature map

@pytest.mark.parametrize("name,out", [("tiny_f32", "f32"), ("b4h8_l2k_bf16", "bf16"), ("b4h8_l2k_bf16", "f32"),
                                      ("h16_l16k_bf16", "bf16"), ("h8_l128k_d128_bf16", "bf16")])
def test_featmap_parity(lib, orc, name, out):
    import torch

    w = ss.WORKLOADS[name].with_(B=1, H=1, L=1000)  # ragged row count (not a multiple of 64)
    _say(f"featmap parity {name} out={out} rows={w.L}")
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    fm = _fm(lib, w, A, G)
    x = q.reshape(-1, w.d)
    phi = lib.featmap(fm, to_dev(x, w.dtype), torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref = orc.featmap(x, A, G, w.eps, w.R, w.m)
    got = to_np(phi)
    err = rownorm_rel(got, ref)
    _say(f"  rownorm rel err {err:.3e}, elementwise {elem_rel(got, ref):.3e}")
    tol = TOL["bf16"] if out == "bf16" else (TOL["f32"] if w.dtype == "f32" else 1e-4)
    assert err < tol
    assert np.all(got > 0)  # strictly positive features


@pytest.mark.parametrize("base,d,R,m,out", [
    ("h16_l16k_bf16", 64, 4, 64, "bf16"),        # bf16 -> bf16, d = 64 (the forward's and backward's map)
    ("h16_l16k_bf16", 64, 5, 32, "bf16"),        # F = 160: the second 128-feature slice is partial
    ("h16_l16k_bf16", 32, 4, 64, "bf16"),        # d = 32, four feature blocks per wave
    ("h8_l128k_d128_bf16", 128, 4, 128, "bf16"),  # d = 128, F = 512
    ("h16_l16k_bf16", 64, 4, 64, "f32"),         # bf16 -> fp32
    ("tiny_f32", 64, 4, 64, "f32"),              # fp32 -> fp32, d = 64
    ("tiny_f32", 128, 4, 128, "f32"),            # fp32 -> fp32, d = 128
])
def test_featmap_large_launches(lib, orc, base, d, R, m, out):
    """Launches past the small-launch size (64-row tiles walked by each workgroup), ragged last tile."""
    import torch

    w = ss.WORKLOADS[base].with_(B=1, H=1, L=40961, d=d, R=R, m=m)
    _say(f"featmap large launch {w.dtype} -> {out} d={d} F={w.F} rows={w.L}")
    q, _, _ = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    fm = _fm(lib, w, A, G)
    x = q.reshape(-1, w.d)
    phi = lib.featmap(fm, to_dev(x, w.dtype), torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref = orc.featmap(x, A, G, w.eps, w.R, w.m)
    got = to_np(phi)
    err = rownorm_rel(got, ref)
    _say(f"  rownorm rel err {err:.3e}")
    assert err < (TOL["bf16"] if out == "bf16" else 1e-4)
    # Positive up to rounding: where |a.xh| is below what the fp32 sum of the
    # bf16 products resolves (about |a| 2^-24), the anchor factor, and with it
    # phi, can come out exactly 0; the true value there is negligible in its row.
    assert np.all(got >= 0)
    zero = got == 0
    if zero.any():
        rel = (ref / ref.max(axis=1, keepdims=True))[zero]
        _say(f"  {int(zero.sum())} exact zeros of {got.size}, oracle there <= {rel.max():.1e} of its row's largest")
        assert rel.max() < 1e-12


def test_featmap_per_head_draws(lib, orc):
    import torch

    w = ss.WORKLOADS["h16_l16k_bf16"].with_(B=1, H=3, L=128)
    q, _, _ = ss.make_qkv(w)
    sets = [ss.make_draws(w, seed=[99, s]) for s in range(2)]
    A = np.stack([s[0] for s in sets])
    G = np.stack([s[1] for s in sets])
    fm = _fm(lib, w, A, G)
    phi = to_np(lib.featmap(fm, to_dev(q.reshape(-1, w.d), w.dtype), torch.float32, rows_per_head=w.L))
    torch.cuda.synchronize()
    for h in range(3):
        ref = orc.featmap(q[0, h], A[h % 2], G[h % 2], w.eps, w.R, w.m)
        assert rownorm_rel(phi[h * w.L:(h + 1) * w.L], ref) < 1e-4


# ----------------------------------------------------------------------------
# chunked causal forward

def _run_fwd(lib, w, q, k, v, A, G, chunk=None, S0=None, z0=None, state=False):
    import torch

    fm = _fm(lib, w, A, G)
    res = lib.chunked_fwd(fm, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), chunk or w.chunk,
                          S0=None if S0 is None else torch.from_numpy(np.float32(S0)).cuda(),
                          z0=None if z0 is None else torch.from_numpy(np.float32(z0)).cuda(), return_state=state)
    torch.cuda.synchronize()
    if state:
        return tuple(to_np(t) for t in res)
    return to_np(res)


@pytest.mark.parametrize("name,L,chunk", [
    ("tiny_f32", 256, 32),       # the tiny fp32 workload as specified
    ("tiny_f32", 200, 32),       # ragged tail
    ("tiny_f32", 256, 1),        # chunk of one token
    ("tiny_f32", 97, 128),       # one partial chunk
    ("b4h8_l2k_bf16", 2048, 64),  # fused MFMA path, F = 96
    ("h16_l16k_bf16", 1000, 64),  # fused MFMA path, F = 256, ragged tail, 1 segment per head
    ("h16_l16k_bf16", 1000, 32),  # wide MFMA path (feature maps in HBM), F = 256
    ("b4h8_l2k_bf16", 500, 32),   # general path in bf16 (F = 96 has no wide variant)
])
def test_chunked_parity(lib, orc, name, L, chunk):
    w = ss.WORKLOADS[name].with_(L=L, chunk=chunk)
    if name == "b4h8_l2k_bf16":
        w = w.with_(B=2, H=4)
    if name == "h16_l16k_bf16":
        w = w.with_(H=3)
    _say(f"chunked parity {name} B={w.B} H={w.H} L={L} chunk={chunk} dtype={w.dtype}")
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    o, S, z = _run_fwd(lib, w, q, k, v, A, G, state=True)
    ro, rS, rz = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m, form="recurrent")
    err = rownorm_rel(o, ro)
    _say(f"  o rownorm rel err {err:.3e} elementwise {elem_rel(o, ro):.3e}; "
         f"S {rownorm_rel(S, rS):.3e} z {rownorm_rel(z[..., None], rz[..., None]):.3e}")
    assert err < TOL[w.dtype]
    assert rownorm_rel(S.reshape(-1, w.dv), rS.reshape(-1, w.dv)) < TOL[w.dtype]
    assert np.max(np.abs(z - rz) / rz) < TOL[w.dtype]
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=TOL[w.dtype], atol=TOL[w.dtype])  # o_1 = v_1


@pytest.mark.parametrize("d,dv,R,m,H,L", [
    (128, 128, 4, 128, 2, 1000),  # the long-sequence shape's head geometry; 32 segments, ragged tail
    (64, 128, 3, 128, 2, 333),    # F = 384
    (128, 64, 2, 64, 3, 77),      # F = 128, dv = 64 (four feature slices per column group)
    (32, 64, 4, 128, 1, 513),     # d = 32, F = 512, dv = 64
    (128, 128, 4, 128, 1, 20),    # one segment, one partial chunk
    (64, 128, 2, 64, 2, 451),     # F = 128, dv = 128
    (32, 128, 4, 64, 2, 390),     # F = 256, dv = 128
    (128, 64, 3, 128, 2, 333),    # F = 384, dv = 64
    (64, 64, 16, 16, 2, 300),     # the most nodes, R = 16 (m = 16 keeps F = 256 off the fused kernels)
])
def test_wide_parity(lib, orc, d, dv, R, m, H, L):
    """The wide MFMA path (feature maps written once in bf16, state kept on chip per segment)."""
    w = ss.WORKLOADS["h8_l128k_d128_bf16"].with_(H=H, L=L, d=d, dv=dv, R=R, m=m)
    _say(f"wide parity d={d} dv={dv} F={w.F} H={H} L={L}")
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    o, S, z = _run_fwd(lib, w, q, k, v, A, G, state=True)
    ro, rS, rz = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m, form="recurrent")
    err = rownorm_rel(o, ro)
    s_err = rownorm_rel(S.reshape(-1, w.dv), rS.reshape(-1, w.dv))
    z_err = float(np.max(np.abs(z - rz) / rz))
    _say(f"  o rownorm rel err {err:.3e}; S {s_err:.3e} z {z_err:.3e}")
    assert err < TOL["bf16"] and s_err < TOL["bf16"] and z_err < TOL["bf16"]
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=TOL["bf16"], atol=TOL["bf16"])  # o_1 = v_1


@pytest.mark.parametrize("R,m,per_head", [
    (2, 16, False),   # F = 32 on the F = 64 kernels
    (3, 16, True),    # F = 48 -> 64, one draw set per head
    (5, 16, False),   # F = 80 -> 96
    (1, 128, False),  # F = 128, built: no padding
    (5, 32, True),    # F = 160 -> 256
    (7, 32, False),   # F = 224 -> 256
    (8, 32, True),    # F = 256, built: eight nodes, one per producer wave
])
def test_fused_padded_features(lib, orc, R, m, per_head):
    """Feature counts the fused kernels are not built for run on zero-padded
    features; the state handoff is at the caller's F (S_out aliasing S0 too)."""
    import torch

    w = ss.WORKLOADS["h16_l16k_bf16"].with_(H=2, L=700, R=R, m=m)
    _say(f"fused padded F={w.F} per_head={per_head}")
    q, k, v = ss.make_qkv(w)
    if per_head:
        draws = [ss.make_draws(w, seed=[3, 80 + h]) for h in range(w.B * w.H)]
        A, G = np.stack([a for a, _ in draws]), np.stack([g for _, g in draws])
    else:
        A, G = ss.make_draws(w)
    cut = 333
    o1, S1, z1 = _run_fwd(lib, w, q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], A, G, state=True)
    assert S1.shape == (w.B * w.H, w.F, w.dv) and z1.shape == (w.B * w.H, w.F)
    fm = _fm(lib, w, A, G)
    S = torch.from_numpy(np.float32(S1)).cuda()
    z = torch.from_numpy(np.float32(z1)).cuda()
    o2 = lib.chunked_fwd(fm, to_dev(q[:, :, cut:], w.dtype), to_dev(k[:, :, cut:], w.dtype),
                         to_dev(v[:, :, cut:], w.dtype), 64, S0=S, z0=z, S_out=S, z_out=z, return_state=True)[0]
    torch.cuda.synchronize()
    ro, rS, rz = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m, form="recurrent", per_head_draws=per_head)
    err = rownorm_rel(np.concatenate([o1, to_np(o2)], axis=2), ro)
    S2, z2 = to_np(S), to_np(z)
    s_err = rownorm_rel(S2.reshape(-1, w.dv), rS.reshape(-1, w.dv))
    z_err = float(np.max(np.abs(z2 - rz) / rz))
    _say(f"  o rownorm rel err {err:.3e}; S {s_err:.3e} z {z_err:.3e}")
    assert err < TOL["bf16"] and s_err < TOL["bf16"] and z_err < TOL["bf16"]


def test_wide_initial_state_and_handoff(lib, orc):
    """Wide path: [0, L1) then [L1, L) with the state carried equals one pass."""
    w = ss.WORKLOADS["h8_l128k_d128_bf16"].with_(H=2, L=900)
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    cut = 416
    o1, S1, z1 = _run_fwd(lib, w, q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], A, G, state=True)
    o2, S2, z2 = _run_fwd(lib, w, q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], A, G, S0=S1, z0=z1, state=True)
    ro, rS, rz = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m, form="recurrent")
    assert rownorm_rel(np.concatenate([o1, o2], axis=2), ro) < TOL["bf16"]
    assert rownorm_rel(S2.reshape(-1, w.dv), rS.reshape(-1, w.dv)) < TOL["bf16"]
    assert np.max(np.abs(z2 - rz) / rz) < TOL["bf16"]


def test_wide_per_head_draws_in_place(lib, orc):
    """Wide path with one draw set per head, the state handed over in place (S_out aliases S0)."""
    import torch

    w = ss.WORKLOADS["h8_l128k_d128_bf16"].with_(H=3, L=700)
    _say(f"wide per-head draws in place F={w.F} H={w.H} L={w.L}")
    q, k, v = ss.make_qkv(w)
    draws = [ss.make_draws(w, seed=[6, 70 + h]) for h in range(w.H)]
    A, G = np.stack([a for a, _ in draws]), np.stack([g for _, g in draws])
    cut = 288
    o1, S1, z1 = _run_fwd(lib, w, q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], A, G, state=True)
    fm = _fm(lib, w, A, G)
    S = torch.from_numpy(np.float32(S1)).cuda()
    z = torch.from_numpy(np.float32(z1)).cuda()
    o2 = lib.chunked_fwd(fm, to_dev(q[:, :, cut:], w.dtype), to_dev(k[:, :, cut:], w.dtype),
                         to_dev(v[:, :, cut:], w.dtype), w.chunk, S0=S, z0=z, S_out=S, z_out=z, return_state=True)[0]
    torch.cuda.synchronize()
    ro, rS, rz = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m, form="recurrent", per_head_draws=True)
    err = rownorm_rel(np.concatenate([o1, to_np(o2)], axis=2), ro)
    s_err = rownorm_rel(to_np(S).reshape(-1, w.dv), rS.reshape(-1, w.dv))
    z_err = float(np.max(np.abs(to_np(z) - rz) / rz))
    _say(f"  o rownorm rel err {err:.3e}; S {s_err:.3e} z {z_err:.3e}")
    assert err < TOL["bf16"] and s_err < TOL["bf16"] and z_err < TOL["bf16"]


def test_chunked_initial_state_and_handoff(lib, orc):
    """Running [0, L1) then [L1, L) with the state carried equals one pass; S_out may alias S0."""
    import torch

    for name in ("tiny_f32", "h16_l16k_bf16"):
        w = ss.WORKLOADS[name].with_(H=2, L=640)
        _say(f"state handoff {name}")
        q, k, v = ss.make_qkv(w)
        A, G = ss.make_draws(w)
        cut = 320 if name != "tiny_f32" else 96
        o1, S1, z1 = _run_fwd(lib, w, q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], A, G, state=True)
        o2, S2, z2 = _run_fwd(lib, w, q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], A, G, S0=S1, z0=z1, state=True)
        ro, rS, rz = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m, form="recurrent")
        got = np.concatenate([o1, o2], axis=2)
        assert rownorm_rel(got, ro) < TOL[w.dtype]
        assert rownorm_rel(S2.reshape(-1, w.dv), rS.reshape(-1, w.dv)) < TOL[w.dtype]
        # in place: S_out aliases S0
        fm = _fm(lib, w, A, G)
        S = torch.from_numpy(np.float32(S1)).cuda()
        z = torch.from_numpy(np.float32(z1)).cuda()
        o3 = lib.chunked_fwd(fm, to_dev(q[:, :, cut:], w.dtype), to_dev(k[:, :, cut:], w.dtype),
                             to_dev(v[:, :, cut:], w.dtype), w.chunk, S0=S, z0=z, S_out=S, z_out=z,
                             return_state=True)[0]
        torch.cuda.synchronize()
        assert rownorm_rel(to_np(o3), ro[:, :, cut:]) < TOL[w.dtype]
        assert rownorm_rel(to_np(S).reshape(-1, w.dv), rS.reshape(-1, w.dv)) < TOL[w.dtype]


def test_chunked_chunk_size_invariance(lib):
    """Chunk size only changes summation order (fp32 general path)."""
    w = ss.WORKLOADS["tiny_f32"].with_(L=300)
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    outs = [_run_fwd(lib, w, q, k, v, A, G, chunk=c) for c in (1, 16, 32, 100, 128)]
    for o in outs[1:]:
        assert rownorm_rel(o, outs[0]) < 1e-5


@pytest.mark.parametrize("R,m", [(4, 64), (5, 16)])  # F = 256, and F = 80 on zero-padded features
def test_chunked_edge_cases(lib, R, m):
    import torch

    w = ss.WORKLOADS["h16_l16k_bf16"].with_(H=2, L=64, R=R, m=m)
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    fm = _fm(lib, w, A, G)
    # L = 0: only the state passes through
    S0 = torch.randn(2, w.F, w.dv, device="cuda").abs()
    z0 = torch.rand(2, w.F, device="cuda") + 0.5
    e = torch.empty(1, 2, 0, w.d, dtype=torch.bfloat16, device="cuda")
    ev = torch.empty(1, 2, 0, w.dv, dtype=torch.bfloat16, device="cuda")
    o, S, z = lib.chunked_fwd(fm, e, e, ev, 64, S0=S0, z0=z0, return_state=True)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(S, S0) and torch.equal(z, z0)
    # B*H = 0
    e0 = torch.empty(0, 2, 64, w.d, dtype=torch.bfloat16, device="cuda")
    lib.chunked_fwd(fm, e0, e0, e0, 64)
    # zero q rows give finite outputs only where the features vanish: the row is 0/0 -> NaN by
    # the method's definition; a zero key simply contributes nothing
    k0 = k.copy()
    k0[:, :, 5] = 0
    o = _run_fwd(lib, w, q, k0, v, A, G)
    assert np.all(np.isfinite(o))


def test_fused_full_size_h16_l16k(lib, orc):
    """The headline workload at full size (B1 H16 L16384, F=256, chunk 64) in the bench's launch
    configuration; two whole heads are checked against the oracle's recurrent form."""
    w = ss.WORKLOADS["h16_l16k_bf16"]
    _say("full size h16_l16k_bf16: GPU forward")
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    o, S, z = _run_fwd(lib, w, q, k, v, A, G, state=True)
    assert np.all(np.isfinite(o))
    for h in (0, 11):
        _say(f"  oracle head {h}")
        ro, rS, rz = orc.slay_causal(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], A, G, w.eps, w.R, w.m)
        err = rownorm_rel(o[:, h:h + 1], ro)
        _say(f"  head {h}: o rownorm rel err {err:.3e}; S {rownorm_rel(S[h], rS[0]):.3e}")
        assert err < TOL["bf16"]
        assert rownorm_rel(S[h], rS[0]) < TOL["bf16"]
    # convex hull invariant on all heads
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    slack = 0.02 * (hi - lo) + 1e-2
    assert np.all(o >= lo - slack) and np.all(o <= hi + slack)


def test_full_size_b4h8_l2k(lib, orc):
    w = ss.WORKLOADS["b4h8_l2k_bf16"]
    _say("full size b4h8_l2k_bf16")
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    o = _run_fwd(lib, w, q, k, v, A, G)
    ro = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m)[0]
    err = rownorm_rel(o, ro)
    _say(f"  o rownorm rel err {err:.3e}")
    assert err < TOL["bf16"]


def test_full_size_h8_l128k_d128_sampled(lib, orc):
    """B1 H8 L131072 d=dv=128, F=512, chunk 128 at full size; sampled rows of two heads are
    checked one by one against the oracle."""
    w = ss.WORKLOADS["h8_l128k_d128_bf16"]
    _say("full size h8_l128k_d128_bf16: GPU forward")
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w)
    o = _run_fwd(lib, w, q, k, v, A, G)
    assert np.all(np.isfinite(o))
    rows = np.array([0, 1, 127, 128, 129, 4095, 65537, w.L - 1])
    for h in (0, 7):
        _say(f"  oracle rows of head {h}")
        phk = orc.featmap(k[0, h], A, G, w.eps, w.R, w.m)
        phq = orc.featmap(q[0, h, rows], A, G, w.eps, w.R, w.m)
        ref = orc.attn_rows(rows, phq, phk, v[0, h])
        err = rownorm_rel(o[0, h, rows], ref)
        _say(f"  head {h}: rownorm rel err {err:.3e}")
        assert err < TOL["bf16"]


# ----------------------------------------------------------------------------
# recurrent decode

def _decode_inputs(w, n_heads, steps):
    qs, ks, vs = [], [], []
    for t in range(steps):
        q, k, v = ss.make_decode_step(w, t, n_heads)
        qs.append(q)
        ks.append(k)
        vs.append(v)
    return np.stack(qs, 1), np.stack(ks, 1), np.stack(vs, 1)  # [n_heads, steps, d]


@pytest.mark.parametrize("n_heads,steps", [(128, 4096), (4096, 3)])
def test_decode_parity(lib, orc, n_heads, steps):
    import torch

    w = ss.WORKLOADS["decode_256x16_f32"]
    _say(f"decode parity heads={n_heads} steps={steps}")
    A, G = ss.make_draws(w)
    q, k, v = _decode_inputs(w, n_heads, steps)
    fm = _fm(lib, w, A, G)
    S = torch.zeros(n_heads, w.F, w.dv, device="cuda")
    z = torch.zeros(n_heads, w.F, device="cuda")
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    outs = torch.empty(n_heads, steps, w.dv, device="cuda")
    for t in range(steps):
        outs[:, t] = lib.recurrent_step(fm, qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(), S, z)
    torch.cuda.synchronize()
    ro, rS, rz = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m, form="recurrent")
    got = to_np(outs)
    err = rownorm_rel(got, ro)
    # the state after `steps` tokens, row by row with the floor (a feature row
    # after few steps holds a handful of phi values and inherits their
    # cancellation); the unfloored and per-head figures are reported
    s_err = rowfloor_rel(to_np(S), rS, heads=n_heads)
    z_err = rowfloor_rel(to_np(z)[..., None], rz[..., None], heads=n_heads)
    _say(f"  o rownorm rel err {err:.3e}; S {s_err:.3e}; z {z_err:.3e}; S unfloored per-row "
         f"{rownorm_rel(to_np(S).reshape(-1, w.dv), rS.reshape(-1, w.dv)):.3e}, per head {headnorm_rel(to_np(S), rS):.3e}")
    assert err < TOL["f32"]
    assert s_err < TOL["f32"]
    assert z_err < TOL["f32"]
    np.testing.assert_allclose(got[:, 0], v[:, 0], rtol=1e-5, atol=1e-5)  # first step from zero state returns v


def test_decode_per_head_draws(lib, orc):
    """Decode with draw sets shared by head groups: head h uses set h % 3."""
    import torch

    w = ss.WORKLOADS["decode_256x16_f32"]
    n_heads, steps, n_sets = 48, 16, 3
    _say(f"decode per-head draws heads={n_heads} steps={steps} sets={n_sets}")
    draws = [ss.make_draws(w, seed=[5, 40 + i]) for i in range(n_sets)]
    A, G = np.stack([a for a, _ in draws]), np.stack([g for _, g in draws])
    q, k, v = _decode_inputs(w, n_heads, steps)
    fm = _fm(lib, w, A, G)
    S = torch.zeros(n_heads, w.F, w.dv, device="cuda")
    z = torch.zeros(n_heads, w.F, device="cuda")
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    outs = torch.empty(n_heads, steps, w.dv, device="cuda")
    for t in range(steps):
        outs[:, t] = lib.recurrent_step(fm, qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(), S, z)
    torch.cuda.synchronize()
    Ah = np.stack([A[h % n_sets] for h in range(n_heads)])
    Gh = np.stack([G[h % n_sets] for h in range(n_heads)])
    ro, rS, rz = orc.slay_causal(q, k, v, Ah, Gh, w.eps, w.R, w.m, form="recurrent", per_head_draws=True)
    err = rownorm_rel(to_np(outs), ro)
    s_err = rowfloor_rel(to_np(S), rS, heads=n_heads)
    z_err = rowfloor_rel(to_np(z)[..., None], rz[..., None], heads=n_heads)
    _say(f"  o rownorm rel err {err:.3e}; S {s_err:.3e}; z {z_err:.3e}")
    assert err < TOL["f32"] and s_err < TOL["f32"] and z_err < TOL["f32"]


def test_decode_continues_prefill(lib, orc):
    """Chunked forward exports (S, z); decode steps continuing from it equal the all-recurrent run."""
    import torch

    w = ss.WORKLOADS["decode_256x16_f32"]
    wf = ss.WORKLOADS["tiny_f32"].with_(R=4, m=64, H=4, L=100)
    A, G = ss.make_draws(w)
    q, k, v = ss.make_qkv(wf)
    fm = _fm(lib, w, A, G)
    _, S, z = lib.chunked_fwd(fm, to_dev(q[:, :, :90], "f32"), to_dev(k[:, :, :90], "f32"),
                              to_dev(v[:, :, :90], "f32"), 32, return_state=True)
    outs = []
    for t in range(90, 100):
        outs.append(to_np(lib.recurrent_step(fm, to_dev(q[0, :, t], "f32"), to_dev(k[0, :, t], "f32"),
                                             to_dev(v[0, :, t], "f32"), S, z)))
    torch.cuda.synchronize()
    ro = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m)[0]
    got = np.stack(outs, 1)
    assert rownorm_rel(got, ro[0, :, 90:]) < TOL["f32"]


def test_decode_graph_replay_matches_eager(lib):
    """Decode steps captured in a HIP graph and replayed several times (with eager work and
    synchronisation between replays) give the same state and outputs as eager calls."""
    import torch

    w = ss.WORKLOADS["decode_256x16_f32"]
    A, G = ss.make_draws(w)
    fm = _fm(lib, w, A, G)
    nh, n_in = 64, 4
    ins = [tuple(to_dev(a, "f32") for a in ss.make_decode_step(w, t, nh)) for t in range(n_in)]
    ws = torch.empty(lib.recurrent_step_workspace_size(fm, nh, w.dv, torch.float32), dtype=torch.uint8,
                     device="cuda")

    def run(S, z, outs):
        for t, (q, k, v) in enumerate(ins):
            lib.recurrent_step(fm, q, k, v, S, z, out=outs[t], workspace=ws)

    S_e = torch.zeros(nh, w.F, w.dv, device="cuda")
    z_e = torch.zeros(nh, w.F, device="cuda")
    outs_e = [torch.empty(nh, w.dv, device="cuda") for _ in range(n_in)]
    S_g, z_g = S_e.clone(), z_e.clone()
    outs_g = [torch.empty(nh, w.dv, device="cuda") for _ in range(n_in)]
    run(S_g, z_g, outs_g)  # warm-up outside the capture
    torch.cuda.synchronize()
    S_g.zero_()
    z_g.zero_()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(S_g, z_g, outs_g)
    torch.cuda.synchronize()
    S_g.zero_()
    z_g.zero_()
    for rep in range(3):
        graph.replay()
        run(S_e, z_e, outs_e)  # eager work between replays
        torch.cuda.synchronize()
        for t in range(n_in):
            assert torch.equal(outs_g[t], outs_e[t]), (rep, t)
        assert torch.equal(S_g, S_e) and torch.equal(z_g, z_e)


@pytest.mark.parametrize("name,L", [("tiny_f32", 200), ("h16_l16k_bf16", 1000)])
def test_orthogonal_draws_parity(lib, orc, name, L):
    """Positive orthogonal random features change only the caller's PRF draws:
    the same kernels, checked against the oracle on orthogonal draws."""
    w = ss.WORKLOADS[name].with_(H=2, L=L)
    _say(f"orthogonal draws parity {name} L={L}")
    q, k, v = ss.make_qkv(w)
    A, G = ss.make_draws(w, orthogonal=True)
    o = _run_fwd(lib, w, q, k, v, A, G)
    ro = orc.slay_causal(q, k, v, A, G, w.eps, w.R, w.m)[0]
    err = rownorm_rel(o, ro)
    _say(f"  causal o rownorm rel err {err:.3e}")
    assert err < TOL[w.dtype]
    fm = _fm(lib, w, A, G)
    on = to_np(lib.noncausal_fwd(fm, to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)))
    rn = orc.slay_noncausal(q, k, v, A, G, w.eps, w.R, w.m)[0]
    assert rownorm_rel(on, rn) < TOL[w.dtype]
