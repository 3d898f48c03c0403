"""GPU parity of the block-outer NSA selection forward (nsa_sel_fwd_fsa) against the
fp64 oracle: the query-outer forward's small shapes and block_idx edge cases, lists
long enough to be split over several workgroups, dense equivalence, exact token
counts with q = 0, set semantics, determinism, workspace reuse, T=8192 with the small
groups (G = 1 and 4) where this form is the faster one, and the T=4096 G=8 and T=32768
G=16 configurations."""
import math

import numpy as np
import pytest
import torch

import oracle
import causal_attention_tiled_amd as cat
from causal_attention_tiled_amd import inputs

from _parity import BF16_REL, assert_lse_close, assert_rows_close
from test_nsa_parity import SMALL, _edge_block_idx

pytestmark = pytest.mark.gpu


def _run(q, k, v, idx, bs, dev, want_lse=True, workspace=None):
    o, lse = cat.nsa_sel_fwd_fsa(q.to(dev), k.to(dev), v.to(dev),
                                 torch.as_tensor(np.ascontiguousarray(idx), dtype=torch.int32).to(dev),
                                 bs, want_lse=want_lse, workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu(), (lse.cpu() if lse is not None else None)


# the next two select every causal block: early blocks have lists of more than 512
# queries, processed by several workgroups; the last two cover the combine kernel's
# remaining layouts (D = 64 with G = 16: two 8-dim pieces per lane; D = 128 with G = 1 and
# 64 slots: four rows per wave, each with a full wave of slots)
FSA_SMALL = SMALL + [(1, 4, 1, 1056, 64, 32, 33), (1, 8, 2, 1280, 128, 64, 20),
                     (1, 16, 1, 256, 64, 32, 4), (1, 2, 2, 2048, 128, 32, 64)]


@pytest.mark.parametrize("shape", FSA_SMALL, ids=lambda s: "B%dHq%dHkv%dT%dD%dbs%dS%d" % s)
def test_fsa_small(gpu, shape):
    B, Hq, Hkv, T, D, bs, S = shape
    print(f"fsa {shape}", flush=True)
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=T + S)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=T + S)
    o, lse = _run(q, k, v, idx, bs, gpu)
    ro, rl = oracle.nsa_ref(q, k, v, idx, bs)
    assert_rows_close(o, ro, BF16_REL, f"fsa {shape}")
    assert_lse_close(lse, rl, f"fsa {shape}")


@pytest.mark.parametrize("D,bs,G", [(128, 64, 8), (64, 32, 2), (128, 128, 16), (64, 128, 3)])
def test_fsa_edge_block_lists(gpu, D, bs, G):
    B, Hkv, T, S = 2, 2, 512, 6
    Hq = Hkv * G
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=3)
    idx = _edge_block_idx(B, Hkv, T, bs, S, seed=3)
    o, lse = _run(q, k, v, idx, bs, gpu)
    ro, rl = oracle.nsa_ref(q, k, v, idx, bs)
    assert_rows_close(o, ro, BF16_REL, "edge block lists")
    assert_lse_close(lse, rl, "edge block lists")
    empty = rl == -1e9
    assert empty.any()
    assert np.all(o.float().numpy()[empty] == 0.0)


def test_fsa_dense_equivalence(gpu):
    """Every causally valid block selected, G = 2: dense causal softmax attention."""
    B, Hkv, G, T, D, bs = 1, 2, 2, 256, 64, 32
    q, k, v = inputs.nsa_inputs(B, Hkv * G, Hkv, T, D, seed=9)
    nblk = T // bs
    idx = np.full((B, Hkv, T, nblk), -1, dtype=np.int32)
    for i in range(T):
        idx[:, :, i, :i // bs + 1] = np.arange(i // bs + 1)
    o, lse = _run(q, k, v, idx, bs, gpu)
    qd = q.double()
    kd = k.double().repeat_interleave(G, dim=1)
    vd = v.double().repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, is_causal=True)
    assert_rows_close(o, ref.numpy(), BF16_REL, "dense equivalence")
    s = (qd @ kd.transpose(-1, -2).contiguous()) / math.sqrt(D)
    s = s.masked_fill(~torch.ones(T, T, dtype=torch.bool).tril(), float("-inf"))
    assert_lse_close(lse, torch.logsumexp(s, -1).numpy(), "dense equivalence")


def test_fsa_zero_q_counts_tokens_exactly(gpu):
    """q = 0: exp(lse) rounds to |A| and, with v = bits of the position, out is the
    exact fraction of A with each bit (catches a block counted twice or missed)."""
    B, Hq, Hkv, T, D, bs, S = 1, 4, 1, 1024, 64, 64, 6
    _, k, _ = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=6)
    q = torch.zeros(B, Hq, T, D, dtype=torch.bfloat16)
    bits = torch.tensor([[(j >> (d % 8)) & 1 for d in range(D)] for j in range(T)],
                        dtype=torch.bfloat16)[None, None]
    idx = _edge_block_idx(B, Hkv, T, bs, S, seed=6)
    o, lse = _run(q, k, bits, idx, bs, gpu)
    ro, rl = oracle.nsa_ref(q, k, bits, idx, bs)
    counts = np.where(rl > -1e9, np.exp(rl), 0.0)
    gcounts = np.where(lse.numpy() > -1e9, np.exp(lse.numpy().astype(np.float64)), 0.0)
    assert np.array_equal(np.rint(gcounts), np.rint(counts))
    assert_rows_close(o, ro, BF16_REL, "zero-q fractions")


def test_fsa_set_semantics_and_determinism(gpu):
    """Repeating slots changes nothing, bit for bit; the same call twice is bit-identical;
    without lse the output is the same."""
    B, Hq, Hkv, T, D, bs, S = 1, 8, 2, 512, 128, 64, 5
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=8)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=8)
    o, lse = _run(q, k, v, idx, bs, gpu)
    o2, lse2 = _run(q, k, v, idx, bs, gpu)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    dup = np.concatenate([idx, idx[..., :3]], axis=-1)
    od, ld = _run(q, k, v, dup, bs, gpu)
    assert torch.equal(o, od) and torch.equal(lse, ld)
    on, ln = _run(q, k, v, idx, bs, gpu, want_lse=False)
    assert ln is None and torch.equal(o, on)


def test_fsa_workspace_reuse(gpu):
    """One workspace for a large call and then a smaller one: the second call sees the
    first one's leftovers and must not depend on them."""
    B, Hq, Hkv, D, bs, S = 1, 8, 2, 128, 64, 8
    big = cat.nsa_sel_fsa_workspace_bytes(B, Hq, Hkv, 1024, D, bs, S)
    ws = torch.full((big,), 0x5A, dtype=torch.uint8, device=gpu)
    for T in (1024, 384):
        q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=T)
        idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=T)
        o, lse = _run(q, k, v, idx, bs, gpu, workspace=ws)
        ro, rl = oracle.nsa_ref(q, k, v, idx, bs)
        assert_rows_close(o, ro, BF16_REL, f"workspace reuse T={T}")
        assert_lse_close(lse, rl, f"workspace reuse T={T}")


def test_fsa_matches_query_outer_T4096_G8(gpu, nsa_c4_case):
    """B=2 Hq=32 Hkv=4 T=4096 D=128 bs=64 S=16: every element against the oracle, and
    every row within the bf16 tolerance of the query-outer kernel."""
    c = nsa_c4_case
    q, k, v, idx, bs = c["q"], c["k"], c["v"], c["idx"], c["c"]["block_size"]
    o, lse = _run(q, k, v, idx, bs, gpu)
    assert_rows_close(o, c["ref_o"], BF16_REL, "fsa T4096 G8")
    assert_lse_close(lse, c["ref_lse"], "fsa T4096 G8")
    oq, lq = cat.nsa_sel_fwd(q.to(gpu), k.to(gpu), v.to(gpu), torch.as_tensor(idx).to(gpu), bs)
    torch.cuda.synchronize()
    assert_rows_close(o, oq.cpu().double().numpy(), 2 * BF16_REL, "fsa vs query-outer")
    assert_lse_close(lse, lq.cpu().double().numpy(), "fsa vs query-outer")


def test_fsa_config_T32768_G16(gpu, nsa_c5_case):
    """B=1 Hq=64 Hkv=4 T=32768 D=128 bs=64 S=16: every element of o and lse against the
    oracle."""
    c = nsa_c5_case
    print("fsa T32768: gpu", flush=True)
    o, lse = _run(c["q"], c["k"], c["v"], c["idx"], c["c"]["block_size"], gpu)
    D = o.shape[-1]
    assert_rows_close(o.reshape(-1, D)[c["rows"]], c["ref_o"], BF16_REL, "fsa T32768 G16")
    assert_lse_close(lse.reshape(-1)[c["rows"]], c["ref_lse"], "fsa T32768 G16")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("Hkv", [16, 4], ids=["G1", "G4"])
def test_fsa_small_groups_T8192(gpu, Hkv):
    """B=1 Hq=16 T=8192 D=128 bs=64 S=16 with G = 1 and G = 4 (block lists as in the
    benchmarked configurations): every element of o and lse against the oracle."""
    B, Hq, T, D, bs, S = 1, 16, 8192, 128, 64, 16
    print(f"fsa T8192 Hkv={Hkv}: inputs", flush=True)
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=Hkv)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=Hkv)
    o, lse = _run(q, k, v, idx, bs, gpu)
    print(f"fsa T8192 Hkv={Hkv}: oracle", flush=True)
    ro, rl = oracle.nsa_ref(q, k, v, idx, bs)
    assert_rows_close(o, ro, BF16_REL, f"fsa T8192 G{Hq // Hkv}")
    assert_lse_close(lse, rl, f"fsa T8192 G{Hq // Hkv}")
