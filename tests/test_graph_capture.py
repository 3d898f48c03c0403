"""Every entry point captured in a HIP graph (through torch.cuda.graph, on the
capturing stream) and replayed several times, with eager calls of the same entry
point and host synchronisations in between: each replay must reproduce the eager
result bit for bit.  The library issues no allocation and no memset (its index and
flags are cleared by fill kernels), so its launches are capturable as they are."""
import numpy as np
import pytest
import torch

import causal_attention_tiled_amd as cat
from causal_attention_tiled_amd import inputs

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _check_graph(fn, outs, scramble):
    """fn() writes into the tensors of outs; scramble() overwrites the same tensors
    with an eager call on other inputs, so a replay that does nothing is caught."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up on the capture stream, as torch asks
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for r in range(REPLAYS):
        scramble()
        torch.cuda.synchronize()
        assert any(not torch.equal(o, x) for o, x in zip(outs, ref)), "scramble changed nothing"
        g.replay()
        torch.cuda.synchronize()
        for o, x in zip(outs, ref):
            assert torch.equal(o, x), f"replay {r} differs from the eager result"


def test_graph_tra_fwd_and_bwd(gpu):
    B, H, T, D = 1, 4, 512, 128
    q, k, v = (x.to(gpu) for x in inputs.tra_inputs(B, H, T, D, seed=1))
    q2, k2, v2 = (x.to(gpu) for x in inputs.tra_inputs(B, H, T, D, seed=2))
    do = torch.randn(B, H, T, D, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).to(gpu)
    out = torch.empty_like(q)
    _check_graph(lambda: cat.tra_fwd(q, k, v, 1.0, 2.0, out=out), [out],
                 lambda: cat.tra_fwd(q2, k2, v2, 1.0, 2.0, out=out))
    g = [torch.empty_like(q) for _ in range(3)]
    _check_graph(lambda: cat.tra_bwd(q, k, v, do, 1.0, 2.0, dq=g[0], dk=g[1], dv=g[2]), g,
                 lambda: cat.tra_bwd(q2, k2, v2, do, 1.0, 2.0, dq=g[0], dk=g[1], dv=g[2]))


def test_graph_tda_fwd(gpu):
    B, H, T, D = 1, 2, 384, 128
    t = [x.to(gpu) for x in inputs.tda_inputs(B, H, T, D, seed=4)]
    t2 = [x.to(gpu) for x in inputs.tda_inputs(B, H, T, D, seed=5)]
    ws = torch.empty(cat.tda_workspace_bytes(B, H, T, D, True), dtype=torch.uint8, device=gpu)
    out = torch.empty_like(t[0])
    _check_graph(lambda: cat.tda_fwd(*t, 0.1, 0.5, 2.0, normalize=True, out=out, workspace=ws),
                 [out],
                 lambda: cat.tda_fwd(*t2, 0.1, 0.5, 2.0, normalize=True, out=out, workspace=ws))


def test_graph_nsa_forwards_and_backward(gpu):
    B, Hq, Hkv, T, D, bs, S = 1, 8, 2, 1024, 128, 64, 8
    q, k, v = (x.to(gpu) for x in inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=6))
    q2, k2, v2 = (x.to(gpu) for x in inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=7))
    idx = torch.as_tensor(inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=6)).to(gpu)
    idx2 = torch.as_tensor(inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=7)).to(gpu)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=gpu)
    _check_graph(lambda: cat.nsa_sel_fwd(q, k, v, idx, bs, out=o, lse=lse), [o, lse],
                 lambda: cat.nsa_sel_fwd(q2, k2, v2, idx2, bs, out=o, lse=lse))
    wsf = torch.empty(cat.nsa_sel_fsa_workspace_bytes(B, Hq, Hkv, T, D, bs, S), dtype=torch.uint8,
                      device=gpu)
    of = torch.empty_like(q)
    lf = torch.empty_like(lse)
    _check_graph(lambda: cat.nsa_sel_fwd_fsa(q, k, v, idx, bs, out=of, lse=lf, workspace=wsf),
                 [of, lf],
                 lambda: cat.nsa_sel_fwd_fsa(q2, k2, v2, idx2, bs, out=of, lse=lf, workspace=wsf))
    # backward on the forward's own outputs (o, lse from the first forward's inputs)
    cat.nsa_sel_fwd(q, k, v, idx, bs, out=o, lse=lse)
    o2, lse2 = cat.nsa_sel_fwd(q2, k2, v2, idx2, bs)
    do = torch.randn(B, Hq, T, D, generator=torch.Generator().manual_seed(8)).to(torch.bfloat16).to(gpu)
    wsb = torch.empty(cat.nsa_sel_bwd_workspace_bytes(B, Hq, Hkv, T, D, bs, S), dtype=torch.uint8,
                      device=gpu)
    g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    _check_graph(lambda: cat.nsa_sel_bwd(q, k, v, idx, bs, o, lse, do, dq=g[0], dk=g[1], dv=g[2],
                                         workspace=wsb), g,
                 lambda: cat.nsa_sel_bwd(q2, k2, v2, idx2, bs, o2, lse2, do, dq=g[0], dk=g[1],
                                         dv=g[2], workspace=wsb))
