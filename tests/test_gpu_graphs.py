"""The forward (fused and wide paths), variable-length forward and backward captured in HIP graphs.

Each call is captured once (with its workspace and outputs preallocated) and
the graph replayed several times, with eager calls of the same entry point
and synchronisation between the replays; every replay must reproduce the
eager result bit for bit (same kernels, same inputs, same summation order).
"""
import numpy as np
import pytest

import slay_synth as ss
from helpers import to_dev

pytestmark = pytest.mark.gpu

W = ss.WORKLOADS["h16_l16k_bf16"]


@pytest.fixture(scope="module")
def lib():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from kernelized_linear_attention_amd import ops

    return ops


def _replay_matches(fn_graph, fn_eager, outs_graph, outs_eager, reps=3):
    import torch

    fn_graph()  # warm-up outside the capture (one-time attribute setting, code loading)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn_graph()
    torch.cuda.synchronize()
    for rep in range(reps):
        for t in outs_graph:
            t.fill_(float("nan")) if t.is_floating_point() else t.zero_()
        graph.replay()
        fn_eager()
        torch.cuda.synchronize()
        for a, b in zip(outs_graph, outs_eager):
            assert torch.equal(a, b), rep


@pytest.mark.parametrize("R,m", [(4, 64), (5, 32)])  # F = 256, and F = 160 on zero-padded features
def test_forward_graph(lib, R, m):
    import torch

    w = W.with_(H=4, L=2000, R=R, m=m)
    q, k, v = (to_dev(x, "bf16") for x in ss.make_qkv(w))
    A, G = ss.make_draws(w)
    fm = lib.FeatureMap(to_dev(A, "bf16"), to_dev(G, "bf16"), w.R, w.m, w.eps)
    ws = torch.empty(lib.chunked_fwd_workspace_size(fm, 1, 4, w.L, w.dv, 64, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    og, oe = torch.empty_like(v), torch.empty_like(v)
    Sg, Se = (torch.empty(4, w.F, w.dv, device="cuda") for _ in range(2))
    zg, ze = (torch.empty(4, w.F, device="cuda") for _ in range(2))
    _replay_matches(lambda: lib.chunked_fwd(fm, q, k, v, 64, out=og, workspace=ws, return_state=True, S_out=Sg,
                                            z_out=zg),
                    lambda: lib.chunked_fwd(fm, q, k, v, 64, out=oe, workspace=ws, return_state=True, S_out=Se,
                                            z_out=ze),
                    [og, Sg, zg], [oe, Se, ze])


@pytest.mark.parametrize("R,m", [(4, 64), (5, 16)])  # F = 256, and F = 80 on zero-padded features
def test_noncausal_graph(lib, R, m):
    import torch

    w = W.with_(H=3, L=1500, R=R, m=m)
    q, k, v = (to_dev(x, "bf16") for x in ss.make_qkv(w))
    qq = q[:, :, :700].contiguous()
    A, G = ss.make_draws(w)
    fm = lib.FeatureMap(to_dev(A, "bf16"), to_dev(G, "bf16"), w.R, w.m, w.eps)
    ws = torch.empty(lib.noncausal_fwd_workspace_size(fm, 1, 3, 700, w.L, w.dv, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    og = torch.empty(1, 3, 700, w.dv, dtype=torch.bfloat16, device="cuda")
    oe = torch.empty_like(og)
    Sg, Se = (torch.empty(3, w.F, w.dv, device="cuda") for _ in range(2))
    zg, ze = (torch.empty(3, w.F, device="cuda") for _ in range(2))
    _replay_matches(lambda: lib.noncausal_fwd(fm, qq, k, v, out=og, workspace=ws, S_out=Sg, z_out=zg,
                                              return_state=True),
                    lambda: lib.noncausal_fwd(fm, qq, k, v, out=oe, workspace=ws, S_out=Se, z_out=ze,
                                              return_state=True),
                    [og, Sg, zg], [oe, Se, ze])


def test_varlen_graph(lib):
    import torch

    lengths = [700, 0, 1300, 1]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64, device="cuda")
    T = int(sum(lengths))
    q, k, v = (to_dev(x[0], "bf16") for x in ss.make_qkv(W.with_(H=2, L=T)))
    A, G = ss.make_draws(W)
    fm = lib.FeatureMap(to_dev(A, "bf16"), to_dev(G, "bf16"), W.R, W.m, W.eps)
    ws = torch.empty(lib.varlen_fwd_workspace_size(fm, len(lengths), 2, T, W.dv, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    og, oe = torch.empty_like(v), torch.empty_like(v)
    Sg, Se = (torch.empty(len(lengths), 2, W.F, W.dv, device="cuda") for _ in range(2))
    zg, ze = (torch.empty(len(lengths), 2, W.F, device="cuda") for _ in range(2))
    _replay_matches(lambda: lib.varlen_fwd(fm, q, k, v, cu, out=og, workspace=ws, return_state=True, S_out=Sg,
                                           z_out=zg),
                    lambda: lib.varlen_fwd(fm, q, k, v, cu, out=oe, workspace=ws, return_state=True, S_out=Se,
                                           z_out=ze),
                    [og, Sg, zg], [oe, Se, ze])


def test_backward_graph(lib):
    import torch

    w = W.with_(H=2, L=1500)
    q, k, v = (to_dev(x, "bf16") for x in ss.make_qkv(w))
    dout = to_dev(ss.make_grads(w)[0], "bf16")
    A, G = ss.make_draws(w)
    fm = lib.FeatureMap(to_dev(A, "bf16"), to_dev(G, "bf16"), w.R, w.m, w.eps)
    ws = torch.empty(lib.chunked_bwd_workspace_size(fm, 1, 2, w.L, w.dv, 64, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    g = [torch.empty_like(x) for x in (q, k, v)] + [torch.empty(2, w.F, w.dv, device="cuda"),
                                                    torch.empty(2, w.F, device="cuda")]
    e = [torch.empty_like(x) for x in g]

    def run(o):
        lib.chunked_bwd(fm, q, k, v, dout, 64, workspace=ws, dq=o[0], dk=o[1], dv=o[2], dS0=o[3], dz0=o[4],
                        state_grad=True)

    _replay_matches(lambda: run(g), lambda: run(e), g, e)


def test_wide_forward_graph(lib):
    """The wide path (feature maps in the workspace, d = dv = 128, F = 512)."""
    import torch

    w = ss.WORKLOADS["h8_l128k_d128_bf16"].with_(H=2, L=1500)
    q, k, v = (to_dev(x, "bf16") for x in ss.make_qkv(w))
    A, G = ss.make_draws(w)
    fm = lib.FeatureMap(to_dev(A, "bf16"), to_dev(G, "bf16"), w.R, w.m, w.eps)
    ws = torch.empty(lib.chunked_fwd_workspace_size(fm, 1, 2, w.L, w.dv, w.chunk, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    og, oe = torch.empty_like(v), torch.empty_like(v)
    Sg, Se = (torch.empty(2, w.F, w.dv, device="cuda") for _ in range(2))
    zg, ze = (torch.empty(2, w.F, device="cuda") for _ in range(2))
    _replay_matches(lambda: lib.chunked_fwd(fm, q, k, v, w.chunk, out=og, workspace=ws, return_state=True, S_out=Sg,
                                            z_out=zg),
                    lambda: lib.chunked_fwd(fm, q, k, v, w.chunk, out=oe, workspace=ws, return_state=True, S_out=Se,
                                            z_out=ze),
                    [og, Sg, zg], [oe, Se, ze])


def test_padded_backward_graph(lib):
    """The backward at F = 96 (features zero-padded to 256, with the padding
    copies of the draws and of the states inside the graph)."""
    import torch

    w = ss.WORKLOADS["b4h8_l2k_bf16"].with_(B=1, H=2, L=700)
    q, k, v = (to_dev(x, "bf16") for x in ss.make_qkv(w))
    dout, dST, dzT = ss.make_grads(w)
    dout = to_dev(dout, "bf16")
    dST, dzT = (torch.from_numpy(np.float32(x)).cuda() for x in (dST, dzT))
    S0 = torch.rand(2, w.F, w.dv, device="cuda")
    z0 = torch.rand(2, w.F, device="cuda") + 0.5
    A, G = ss.make_draws(w)
    fm = lib.FeatureMap(to_dev(A, "bf16"), to_dev(G, "bf16"), w.R, w.m, w.eps)
    ws = torch.empty(lib.chunked_bwd_workspace_size(fm, 1, 2, w.L, w.dv, 64, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    g = [torch.empty_like(x) for x in (q, k, v)] + [torch.empty(2, w.F, w.dv, device="cuda"),
                                                    torch.empty(2, w.F, device="cuda")]
    e = [torch.empty_like(x) for x in g]

    def run(o):
        lib.chunked_bwd(fm, q, k, v, dout, 64, S0=S0, z0=z0, dS_T=dST, dz_T=dzT, workspace=ws, dq=o[0], dk=o[1],
                        dv=o[2], dS0=o[3], dz0=o[4], state_grad=True)

    _replay_matches(lambda: run(g), lambda: run(e), g, e)
