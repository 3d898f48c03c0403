"""GPU parity of the NSA selection forward (nsa_sel_fwd) against the fp64 oracle
on the same seeded inputs and block lists, the block_idx edge cases, and
GPU-only invariants (group sharing, set semantics, exact empty rows)."""
import math

import numpy as np
import pytest
import torch

import oracle
import causal_attention_tiled_amd as cat
from causal_attention_tiled_amd import inputs

from _parity import BF16_REL, assert_lse_close, assert_rows_close

pytestmark = pytest.mark.gpu


def _run(q, k, v, idx, bs, dev, want_lse=True):
    o, lse = cat.nsa_sel_fwd(q.to(dev), k.to(dev), v.to(dev),
                             torch.as_tensor(np.ascontiguousarray(idx), dtype=torch.int32).to(dev),
                             bs, want_lse=want_lse)
    torch.cuda.synchronize()
    return o.cpu(), (lse.cpu() if lse is not None else None)


SMALL = [  # B, Hq, Hkv, T, D, bs, S
    (1, 8, 2, 256, 128, 64, 4),
    (2, 4, 4, 128, 64, 32, 3),      # G = 1
    (1, 16, 1, 512, 128, 64, 8),    # G = 16
    (1, 6, 2, 256, 128, 128, 2),    # block 128, G = 3
    (1, 3, 1, 64, 64, 64, 1),       # one block, S = 1
    (2, 10, 2, 320, 64, 32, 16),    # G = 5, many slots
    (1, 4, 2, 2048, 64, 32, 64),    # S = 64, the most slots (one per lane): every block
    (1, 4, 2, 96, 128, 32, 2),      # D = 128 with 32-key blocks: one chunk per block
    (2, 8, 1, 384, 128, 64, 1),     # S = 1: only the own block (one or two chunks per query)
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dHq%dHkv%dT%dD%dbs%dS%d" % s)
def test_nsa_small(gpu, shape):
    B, Hq, Hkv, T, D, bs, S = shape
    print(f"nsa {shape}", flush=True)
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=T + S)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=T + S)
    o, lse = _run(q, k, v, idx, bs, gpu)
    ro, rl = oracle.nsa_ref(q, k, v, idx, bs)
    assert_rows_close(o, ro, BF16_REL, f"nsa {shape}")
    assert_lse_close(lse, rl, f"nsa {shape}")


def _edge_block_idx(B, Hkv, T, bs, S, seed):
    """Rows mixing padding, duplicates, future blocks, out-of-range ids and
    all-padding rows."""
    rng = np.random.default_rng(seed)
    nblk = T // bs
    idx = rng.integers(-3, nblk + 3, size=(B, Hkv, T, S)).astype(np.int32)
    idx[..., 1] = idx[..., 0]                                       # duplicates
    idx[:, :, ::7, :] = -1                                          # all padding
    idx[:, :, 3::11, :] = nblk + 4                                  # all past the end
    for i in range(5, T, 13):                                       # all in the future
        idx[:, :, i, :] = min(i // bs + 1, nblk - 1) if i // bs + 1 < nblk else -1
    return idx


@pytest.mark.parametrize("D,bs,G", [(128, 64, 8), (64, 32, 2), (128, 128, 16)])
def test_nsa_edge_block_lists(gpu, D, bs, G):
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
    assert np.all(o.float().numpy()[empty] == 0.0)                  # exactly zero rows


def test_nsa_without_lse(gpu):
    B, Hq, Hkv, T, D, bs, S = 1, 8, 2, 256, 128, 64, 4
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=5)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=5)
    o, lse = _run(q, k, v, idx, bs, gpu, want_lse=False)
    assert lse is None
    o2, _ = _run(q, k, v, idx, bs, gpu)
    assert torch.equal(o, o2)


def test_nsa_zero_q_counts_tokens_exactly(gpu):
    """q = 0: uniform weights over A, so exp(lse) rounds to |A| and, with
    v[j, d] = bit d of (j mod 256), out[d] is the fraction of A with that bit."""
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


def test_nsa_group_heads_bitidentical(gpu):
    """Two heads of a group with the same query give bit-identical rows."""
    B, Hkv, G, T, D, bs, S = 1, 2, 8, 512, 128, 64, 8
    q, k, v = inputs.nsa_inputs(B, Hkv * G, Hkv, T, D, seed=7)
    q[:, 3] = q[:, 0]
    q[:, 15] = q[:, 9]
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=7)
    o, lse = _run(q, k, v, idx, bs, gpu)
    assert torch.equal(o[:, 3], o[:, 0]) and torch.equal(lse[:, 3], lse[:, 0])
    assert torch.equal(o[:, 15], o[:, 9]) and torch.equal(lse[:, 15], lse[:, 9])


def test_nsa_slot_set_semantics(gpu):
    """The selection is a set: repeating slots or permuting them changes nothing, bit for
    bit (the kernel visits the kept blocks in decreasing block order, whatever the slot
    order); both results also match the oracle."""
    B, Hq, Hkv, T, D, bs, S = 1, 8, 2, 512, 128, 64, 5
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=8)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=8)
    o, lse = _run(q, k, v, idx, bs, gpu)
    dup = np.concatenate([idx, idx[..., :3]], axis=-1)
    od, ld = _run(q, k, v, dup, bs, gpu)
    assert torch.equal(o, od) and torch.equal(lse, ld)
    rng = np.random.default_rng(0)
    perm = np.argsort(rng.random(dup.shape), axis=-1)
    op, lp = _run(q, k, v, np.take_along_axis(dup, perm, axis=-1), bs, gpu)
    assert torch.equal(op, o) and torch.equal(lp, lse)
    ro, rl = oracle.nsa_ref(q, k, v, idx, bs)
    assert_rows_close(o, ro, BF16_REL, "set semantics")
    assert_lse_close(lse, rl, "set semantics")


def test_nsa_dense_equivalence_G1(gpu):
    """Every causally valid block selected, G = 1: dense causal softmax attention."""
    B, H, T, D, bs = 1, 2, 256, 64, 32
    q, k, v = inputs.nsa_inputs(B, H, H, T, D, seed=9)
    nblk = T // bs
    idx = np.full((B, H, T, nblk), -1, dtype=np.int32)
    for i in range(T):
        idx[:, :, i, :i // bs + 1] = np.arange(i // bs + 1)
    o, lse = _run(q, k, v, idx, bs, gpu)
    qd, kd, vd = q.double(), k.double(), v.double()
    ref = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, is_causal=True)
    assert_rows_close(o, ref.numpy(), BF16_REL, "dense equivalence")
    s = (qd @ kd.transpose(-1, -2).contiguous()) / math.sqrt(D)
    s = s.masked_fill(~torch.ones(T, T, dtype=torch.bool).tril(), float("-inf"))
    assert_lse_close(lse, torch.logsumexp(s, -1).numpy(), "dense equivalence")


def test_nsa_config_T4096_G8(gpu, nsa_c4_case):
    """B=2 Hq=32 Hkv=4 T=4096 D=128 bs=64 S=16: every element of o and lse against the
    oracle's full output."""
    c = nsa_c4_case
    print("nsa T4096: gpu", flush=True)
    o, lse = _run(c["q"], c["k"], c["v"], c["idx"], c["c"]["block_size"], gpu)
    assert_rows_close(o, c["ref_o"], BF16_REL, "T4096 G8")
    assert_lse_close(lse, c["ref_lse"], "T4096 G8")


def test_nsa_config_T32768_G16(gpu, nsa_c5_case):
    """B=1 Hq=64 Hkv=4 T=32768 D=128 bs=64 S=16 (the benchmarked launch): every element
    of o and lse (2,097,152 rows) against the oracle."""
    c = nsa_c5_case
    print("nsa T32768: gpu", flush=True)
    o, lse = _run(c["q"], c["k"], c["v"], c["idx"], c["c"]["block_size"], gpu)
    D = o.shape[-1]
    assert_rows_close(o.reshape(-1, D)[c["rows"]], c["ref_o"], BF16_REL, "T32768 G16")
    assert_lse_close(lse.reshape(-1)[c["rows"]], c["ref_lse"], "T32768 G16")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_nsa_long_T131072_G16_sampled_rows(gpu):
    """B=1 Hq=16 Hkv=1 T=131072 D=128 bs=64 S=16 (2048 blocks): o and lse of both forwards
    on every head at the first four query positions, one in 512 and the last 64."""
    import test_nsa_fsa_parity as fsa
    B, Hq, Hkv, T, D, bs, S = 1, 16, 1, 131072, 128, 64, 16
    print("nsa T131072: inputs", flush=True)
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=21)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=21)
    pos = np.unique(np.concatenate([np.arange(4), np.arange(7, T, 512), np.arange(T - 64, T)]))
    rows = (np.arange(B * Hq)[:, None] * T + pos[None, :]).reshape(-1)
    ro, rl = oracle.nsa_ref(q, k, v, idx, bs, rows=rows)
    for name, run in (("query-outer", _run), ("block-outer", fsa._run)):
        print(f"nsa T131072: {name}", flush=True)
        o, lse = run(q, k, v, idx, bs, gpu)
        assert_rows_close(o.reshape(-1, D)[rows], ro, BF16_REL, f"nsa T131072 {name}")
        assert_lse_close(lse.reshape(-1)[rows], rl, f"nsa T131072 {name}")
