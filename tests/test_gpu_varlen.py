"""GPU parity of the variable-length causal forward (sequences of different
lengths packed per head) through the C ABI against the fp64 oracle, which
runs each sequence on its own.  Bar as for the causal forward: 2e-2
row-normwise for bf16, the final states row by row, floored at a tenth of
the (sequence, head)'s rms row norm (helpers.rowfloor_rel).
"""
import sys

import numpy as np
import pytest

import slay_synth as ss
from helpers import TOL, rowfloor_rel, rownorm_rel, to_dev, to_np

pytestmark = pytest.mark.gpu

W = ss.WORKLOADS["h16_l16k_bf16"]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from kernelized_linear_attention_amd import ops

    return ops


def _srel(S, rS, w):
    """States [n_seqs, H, F, dv]: per-row error, floored per (sequence, head)."""
    n = S.size // (w.F * w.dv)
    return rowfloor_rel(S.reshape(n, w.F, w.dv), rS.reshape(n, w.F, w.dv), heads=n)


def _zrel(z, rz, w):
    n = z.size // w.F
    return rowfloor_rel(z.reshape(n, w.F, 1), rz.reshape(n, w.F, 1), heads=n)


def _packed(H, lengths, seed):
    """q, k [H, T, d], v [H, T, dv] (bf16-exact) and the offsets of the sequences."""
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1])
    q, k, v = ss.make_qkv(W.with_(B=1, H=H, L=max(T, 1)), seed=seed)
    return q[0, :, :T], k[0, :, :T], v[0, :, :T], cu


def _states(n, H, seed, w=W):
    rng = np.random.default_rng(seed)
    S0 = np.abs(rng.standard_normal((n, H, w.F, w.dv))).astype(np.float32)
    z0 = (rng.random((n, H, w.F)) + 0.5).astype(np.float32)
    return S0, z0


def _run(lib, q, k, v, cu, A, G, S0=None, z0=None, out=None, w=W):
    import torch

    fm = lib.FeatureMap(to_dev(A, "bf16"), to_dev(G, "bf16"), w.R, w.m, w.eps)
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    o, S, z = lib.varlen_fwd(fm, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                             torch.from_numpy(cu).cuda(), S0=f32(S0), z0=f32(z0), return_state=True, out=out)
    torch.cuda.synchronize()
    return to_np(o), to_np(S), to_np(z)


@pytest.mark.parametrize("H,lengths,with_state", [
    (2, [300, 0, 1, 1000, 77, 2049, 128], True),   # empty, one-token, ragged and multi-segment sequences
    (3, [64, 64, 64], False),
    (1, [5000], True),
    # 16 heads: segments of 1024 tokens; the tails 512, 256, 256 share one work item (a pack),
    # and five sequences end with a whole segment that writes their final state
    (16, [6144, 4096, 2048, 2048, 1024, 512, 256, 256], True),
])
def test_varlen_parity(lib, orc, H, lengths, with_state):
    _say(f"varlen parity H={H} lengths={lengths} state={with_state}")
    q, k, v, cu = _packed(H, lengths, [3, 70, len(lengths)])
    A, G = ss.make_draws(W)
    S0, z0 = _states(len(lengths), H, 5) if with_state else (None, None)
    o, S, z = _run(lib, q, k, v, cu, A, G, S0, z0)
    ro, rS, rz = orc.slay_causal_varlen(q, k, v, cu, A, G, W.eps, W.R, W.m, S0=S0, z0=z0)
    nz = [s for s, n in enumerate(lengths) if n > 0]
    err = rownorm_rel(o, ro) if cu[-1] > 0 else 0.0
    s_err = _srel(S, rS, W)
    z_err = _zrel(z, rz, W)
    _say(f"  o rownorm {err:.3e}; S {s_err:.3e} z {z_err:.3e} (non-empty sequences {nz})")
    assert err < TOL["bf16"] and s_err < TOL["bf16"] and z_err < TOL["bf16"]
    for s, n in enumerate(lengths):  # an empty sequence passes its state through unchanged
        if n == 0:
            assert np.array_equal(S[s], np.float32(S0[s]) if with_state else np.zeros_like(S[s]))


def test_varlen_equal_lengths_match_dense(lib):
    """Equal lengths are a dense batch: the packed call matches slay_attn_chunked_fwd on [B][H][L]."""
    import torch

    B, H, L = 4, 2, 512
    q, k, v, cu = _packed(H, [L] * B, [3, 71])
    A, G = ss.make_draws(W)
    o, S, z = _run(lib, q, k, v, cu, A, G)
    fm = lib.FeatureMap(to_dev(A, "bf16"), to_dev(G, "bf16"), W.R, W.m, W.eps)
    dense = lambda x: to_dev(np.ascontiguousarray(x.reshape(H, B, L, -1).transpose(1, 0, 2, 3)), "bf16")
    od, Sd, zd = lib.chunked_fwd(fm, dense(q), dense(k), dense(v), 64, return_state=True)
    torch.cuda.synchronize()
    od = to_np(od).transpose(1, 0, 2, 3).reshape(H, B * L, -1)
    assert rownorm_rel(o, od) < 1e-2
    assert _srel(S, to_np(Sd).reshape(B, H, W.F, W.dv), W) < 1e-4


def test_varlen_prefill_then_decode(lib, orc):
    """The final states of a mixed-length prefill are the decode state of every (sequence, head)."""
    import torch

    H, lengths = 2, [200, 37, 513]
    q, k, v, cu = _packed(H, lengths, [3, 72])
    A, G = ss.make_draws(W)
    _, S, z = _run(lib, q, k, v, cu, A, G)
    n = len(lengths) * H
    fm = lib.FeatureMap(to_dev(A, "bf16"), to_dev(G, "bf16"), W.R, W.m, W.eps)
    Sd = torch.from_numpy(np.float32(S.reshape(n, W.F, W.dv))).cuda()
    zd = torch.from_numpy(np.float32(z.reshape(n, W.F))).cuda()
    rng = np.random.default_rng(9)
    steps = [tuple(ss.bf16_round(rng.standard_normal((n, x)).astype(np.float32)) for x in (W.d, W.d, W.dv))
             for _ in range(5)]
    for qs, ks, vs in steps:
        o_last = lib.recurrent_step(fm, to_dev(qs, "bf16"), to_dev(ks, "bf16"), to_dev(vs, "bf16"), Sd, zd)
    torch.cuda.synchronize()
    # oracle: each sequence's prompt plus the five decode tokens as one causal sequence
    for s, L in enumerate(lengths):
        b = int(cu[s])
        for h in range(H):
            row = s * H + h
            qq = np.concatenate([q[h, b:b + L]] + [st[0][row:row + 1] for st in steps])
            kk = np.concatenate([k[h, b:b + L]] + [st[1][row:row + 1] for st in steps])
            vv = np.concatenate([v[h, b:b + L]] + [st[2][row:row + 1] for st in steps])
            ro, _, _ = orc.slay_causal(qq[None], kk[None], vv[None], A, G, W.eps, W.R, W.m)
            assert rownorm_rel(to_np(o_last)[row:row + 1], ro[0, -1:]) < TOL["bf16"]


@pytest.mark.parametrize("n_seqs,max_len,H", [
    (300, 90, 1),    # the work list stages offsets and tails in LDS (up to 2048 sequences)
    (2100, 9, 1),    # more sequences: the work list reads them from memory
])
def test_varlen_many_short_sequences(lib, orc, n_seqs, max_len, H):
    """Many short sequences: their tails share work items (packs of many pieces)."""
    _say(f"varlen many short sequences n={n_seqs} max_len={max_len} H={H}")
    rng = np.random.default_rng([11, n_seqs])
    lengths = [int(x) for x in rng.integers(0, max_len, n_seqs)]
    q, k, v, cu = _packed(H, lengths, [3, 73, n_seqs])
    A, G = ss.make_draws(W)
    S0, z0 = _states(n_seqs, H, 7)
    o, S, z = _run(lib, q, k, v, cu, A, G, S0, z0)
    ro, rS, rz = orc.slay_causal_varlen(q, k, v, cu, A, G, W.eps, W.R, W.m, S0=S0, z0=z0)
    err, s_err, z_err = rownorm_rel(o, ro), _srel(S, rS, W), _zrel(z, rz, W)
    _say(f"  o rownorm {err:.3e}; S {s_err:.3e} z {z_err:.3e}")
    assert err < TOL["bf16"] and s_err < TOL["bf16"] and z_err < TOL["bf16"]


@pytest.mark.parametrize("R,m", [(4, 64), (3, 32)])  # F = 256, and F = 96 on zero-padded features
def test_varlen_bad_offsets_compute_nothing(lib, R, m):
    """Offsets that decrease, or do not end at the token count, give no work:
    o keeps its contents and the final states are the initial ones."""
    import torch

    w = W.with_(R=R, m=m)
    H = 2
    q, k, v, _ = _packed(H, [100, 100], [3, 74])
    A, G = ss.make_draws(w)
    S0, z0 = _states(2, H, 6, w)
    for cu in (np.array([0, 150, 120], np.int64), np.array([0, 100, 150], np.int64)):
        out = torch.full((H, 200, w.dv), 7.0, dtype=torch.bfloat16, device="cuda")
        o, S, z = _run(lib, q, k, v, cu, A, G, S0, z0, out=out, w=w)
        assert np.all(o == 7.0)
        assert np.array_equal(S, np.float32(S0)) and np.array_equal(z, np.float32(z0))


def test_varlen_no_sequences_and_unsupported(lib):
    import torch

    fm = lib.FeatureMap(to_dev(np.zeros((W.F, W.d)), "bf16"), to_dev(np.zeros((W.F, W.d)), "bf16"), W.R, W.m, W.eps)
    e = torch.empty(2, 0, W.d, dtype=torch.bfloat16, device="cuda")
    lib.varlen_fwd(fm, e, e, e, torch.zeros(1, dtype=torch.int64, device="cuda"))
    fm64 = lib.FeatureMap(to_dev(np.zeros((64, W.d)), "bf16"), to_dev(np.zeros((64, W.d)), "bf16"), 4, 16, W.eps)
    x = torch.zeros(1, 64, W.d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(Exception, match="variable-length"):  # m = 16: a wave's feature blocks would span two nodes
        lib.varlen_fwd(fm64, x, x, x, torch.tensor([0, 64], dtype=torch.int64, device="cuda"))


@pytest.mark.parametrize("R,m,per_head", [(3, 32, False), (5, 32, True), (1, 32, False)])
def test_varlen_padded_features(lib, orc, R, m, per_head):
    """Feature counts below 256 run on zero-padded features: initial states in,
    final states out at the caller's F, one draw set per head or shared."""
    import torch

    w = W.with_(R=R, m=m)
    H, lengths = 2, [300, 0, 77, 1500, 64]
    _say(f"varlen padded F={w.F} per_head={per_head}")
    q, k, v, cu = _packed(H, lengths, [3, 75])
    if per_head:
        draws = [ss.make_draws(w, seed=[3, 90 + h]) for h in range(H)]
        A, G = np.stack([a for a, _ in draws]), np.stack([g for _, g in draws])
    else:
        A, G = ss.make_draws(w)
    rng = np.random.default_rng(8)
    S0 = np.abs(rng.standard_normal((len(lengths), H, w.F, w.dv))).astype(np.float32)
    z0 = (rng.random((len(lengths), H, w.F)) + 0.5).astype(np.float32)
    fm = lib.FeatureMap(to_dev(A, "bf16"), to_dev(G, "bf16"), R, m, w.eps)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    o, S, z = lib.varlen_fwd(fm, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                             torch.from_numpy(cu).cuda(), S0=f32(S0), z0=f32(z0), return_state=True)
    torch.cuda.synchronize()
    o, S, z = to_np(o), to_np(S), to_np(z)
    assert S.shape == (len(lengths), H, w.F, w.dv) and z.shape == (len(lengths), H, w.F)
    if per_head:  # the oracle takes one head's draws at a time
        outs = [orc.slay_causal_varlen(q[h:h + 1], k[h:h + 1], v[h:h + 1], cu, A[h], G[h], w.eps, R, m,
                                       S0=S0[:, h:h + 1], z0=z0[:, h:h + 1]) for h in range(H)]
        ro = np.concatenate([x[0] for x in outs], axis=0)
        rS = np.concatenate([x[1] for x in outs], axis=1)
        rz = np.concatenate([x[2] for x in outs], axis=1)
    else:
        ro, rS, rz = orc.slay_causal_varlen(q, k, v, cu, A, G, w.eps, R, m, S0=S0, z0=z0)
    err = rownorm_rel(o, ro)
    s_err = _srel(S, rS, w)
    z_err = _zrel(z, rz, w)
    _say(f"  o rownorm {err:.3e}; S {s_err:.3e} z {z_err:.3e}")
    assert err < TOL["bf16"] and s_err < TOL["bf16"] and z_err < TOL["bf16"]
    assert np.array_equal(S[1], S0[1]) and np.array_equal(z[1], z0[1])  # the empty sequence
