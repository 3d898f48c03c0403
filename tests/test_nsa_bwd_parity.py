"""GPU parity of the NSA selection-branch backward (nsa_sel_bwd) against the fp64
oracle on the same seeded inputs: small shapes and the T=4096 G=8 configuration on every
element, the T=32768 G=16 configuration on a dense slice (every head at one query position
in 8, every kv head at one key position in 8); plus determinism, set semantics and rows or
blocks that nothing attends."""
import numpy as np
import pytest
import torch

import oracle
import causal_attention_tiled_amd as cat
from causal_attention_tiled_amd import inputs

from _parity import BF16_REL, assert_rows_close, sample_rows

pytestmark = pytest.mark.gpu

# A query that attends a single key has dq = 0 exactly (P = 1, dP - delta = 0); the
# kernel's P = exp(s - lse) carries the fp32 rounding of the forward's lse, so it
# leaves a residue near 1e-7 * |dP| * |k|.  Those dq rows, and only those, are held to
# an absolute floor of 1e-4 of the largest gradient in the compared tensor.
FLOOR = 1e-4


def _single_key_rows(idx, bs, G):
    """[B, Hq, T] flags: query (b, h, i) attends exactly one key (its set of distinct
    in-range selected blocks, cut at position i, holds one token)."""
    idx = np.asarray(idx)
    B, Hkv, T, S = idx.shape
    nblk = T // bs
    i = np.arange(T)[None, None, :, None]
    blk = np.sort(idx, axis=-1)
    first = np.ones_like(blk, dtype=bool)
    first[..., 1:] = blk[..., 1:] != blk[..., :-1]
    ok = first & (blk >= 0) & (blk < nblk) & (blk * bs <= i)
    ntok = np.where(ok, np.minimum(bs, i - blk * bs + 1), 0).sum(axis=-1)
    return np.repeat(ntok == 1, G, axis=1)


def _dout(shape, seed):
    return torch.randn(*shape, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)


def _run(q, k, v, idx, bs, do, dev):
    gq, gk, gv, gi, gdo = q.to(dev), k.to(dev), v.to(dev), torch.as_tensor(idx).to(dev), do.to(dev)
    o, lse = cat.nsa_sel_fwd(gq, gk, gv, gi, bs)
    g = cat.nsa_sel_bwd(gq, gk, gv, gi, bs, o, lse, gdo)
    torch.cuda.synchronize()
    return [x.cpu() for x in g]


# The last two select every causal block, so the early blocks are attended by more than
# 512 queries and their dk/dv is summed from several workgroups' partial results.
SMALL = [(1, 8, 2, 256, 128, 64, 4), (1, 4, 4, 128, 64, 32, 3), (2, 6, 2, 192, 128, 64, 5),
         (1, 16, 1, 512, 128, 128, 8), (1, 8, 2, 256, 64, 64, 16), (1, 2, 1, 64, 128, 32, 2),
         (1, 4, 1, 1056, 64, 32, 33), (1, 8, 2, 1280, 128, 64, 20)]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: "B%dHq%dHkv%dT%dD%dbs%dS%d" % c)
def test_nsa_bwd_small(gpu, cfg):
    B, Hq, Hkv, T, D, bs, S = cfg
    print(f"nsa_bwd {cfg}", flush=True)
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=T + S)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=S)
    do = _dout((B, Hq, T, D), seed=T)
    got = _run(q, k, v, idx, bs, do, gpu)
    ref = oracle.nsa_bwd_ref(q, k, v, idx, bs, do)
    one = _single_key_rows(idx, bs, Hq // Hkv)
    assert_rows_close(got[0], ref[0], BF16_REL, f"dq {cfg}", floor=FLOOR, floor_rows=one)
    assert_rows_close(got[1], ref[1], BF16_REL, f"dk {cfg}")
    assert_rows_close(got[2], ref[2], BF16_REL, f"dv {cfg}")


def test_nsa_bwd_S64_max_slots(gpu):
    """S = 64, the most slots (one per lane), selecting every causal block: dq on every
    row, dk and dv on sampled key rows (the oracle's key-row gradients sum over every
    query and head, so all 4096 would take minutes)."""
    B, Hq, Hkv, T, D, bs, S = 1, 4, 2, 2048, 64, 32, 64
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=64)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=64)
    do = _dout((B, Hq, T, D), seed=65)
    dq, dk, dv = _run(q, k, v, idx, bs, do, gpu)
    krows = sample_rows(B, Hkv, T, 24, seed=66, extra_positions=(0, 31, 32, 1023, 2047))
    rq, rk, rv = oracle.nsa_bwd_ref(q, k, v, idx, bs, do, krows=krows)
    assert_rows_close(dq, rq, BF16_REL, "dq S64", floor=FLOOR,
                      floor_rows=_single_key_rows(idx, bs, Hq // Hkv))
    assert_rows_close(dk.reshape(-1, D)[krows], rk, BF16_REL, "dk S64")
    assert_rows_close(dv.reshape(-1, D)[krows], rv, BF16_REL, "dv S64")


def test_nsa_bwd_edge_blocks(gpu):
    """Duplicates, out-of-range ids, padding-only rows and unselected blocks."""
    B, Hq, Hkv, T, D, bs, S = 1, 4, 2, 256, 128, 32, 6
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=5)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=5)
    idx[..., 4] = idx[..., 0]            # repeat of the own block
    idx[..., 5] = T // bs + 3            # past the last block
    idx[0, 0, 100:140] = -1              # rows with no block at all
    idx[0, 1, :, 1:] = -1                # kv group 1: own block only
    do = _dout((B, Hq, T, D), seed=6)
    got = _run(q, k, v, idx, bs, do, gpu)
    ref = oracle.nsa_bwd_ref(q, k, v, idx, bs, do)
    assert_rows_close(got[0], ref[0], BF16_REL, "dq edge", floor=FLOOR,
                      floor_rows=_single_key_rows(idx, bs, Hq // Hkv))
    assert_rows_close(got[1], ref[1], BF16_REL, "dk edge")
    assert_rows_close(got[2], ref[2], BF16_REL, "dv edge")
    assert torch.all(got[0][0, 0:2, 100:140] == 0)


def test_nsa_bwd_deterministic(gpu):
    B, Hq, Hkv, T, D, bs, S = 1, 16, 2, 1024, 128, 64, 16
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=7)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=7)
    do = _dout((B, Hq, T, D), seed=8)
    a = _run(q, k, v, idx, bs, do, gpu)
    b = _run(q, k, v, idx, bs, do, gpu)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_nsa_bwd_slot_set_semantics(gpu):
    """The selection is a set: repeating or permuting the slots leaves dq, dk and dv
    unchanged bit for bit (dq visits the kept blocks in decreasing block order, dk/dv
    walk the inverted lists), and the result matches the oracle."""
    B, Hq, Hkv, T, D, bs, S = 1, 8, 2, 512, 128, 64, 5
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=9)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=9)
    do = _dout((B, Hq, T, D), seed=10)
    a = _run(q, k, v, idx, bs, do, gpu)
    dup = np.concatenate([idx, idx[..., :3]], axis=-1)
    perm = np.argsort(np.random.default_rng(1).random(dup.shape), axis=-1)
    b = _run(q, k, v, np.ascontiguousarray(np.take_along_axis(dup, perm, axis=-1)), bs, do, gpu)
    for name, x, y in zip(("dq", "dk", "dv"), a, b):
        assert torch.equal(x, y), f"{name} depends on the slot order"
    ref = oracle.nsa_bwd_ref(q, k, v, idx, bs, do)
    assert_rows_close(a[0], ref[0], BF16_REL, "dq set", floor=FLOOR,
                      floor_rows=_single_key_rows(idx, bs, Hq // Hkv))
    assert_rows_close(a[1], ref[1], BF16_REL, "dk set")
    assert_rows_close(a[2], ref[2], BF16_REL, "dv set")


def test_nsa_bwd_T4096_G8_all_rows(gpu):
    """B=2 Hq=32 Hkv=4 T=4096 D=128 bs=64 S=16: every element of dq, dk and dv against the
    oracle."""
    c = inputs.CONFIGS["nsa_bf16_T4096_G8"]
    B, Hq, Hkv, T, D, bs, S = c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["block_size"], c["S"]
    print("nsa_bwd T4096: inputs", flush=True)
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=0)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=0)
    do = _dout((B, Hq, T, D), seed=1)
    dq, dk, dv = _run(q, k, v, idx, bs, do, gpu)
    print("nsa_bwd T4096: oracle on every row", flush=True)
    rq, rk, rv = oracle.nsa_bwd_ref(q, k, v, idx, bs, do)
    assert_rows_close(dq, rq, BF16_REL, "dq T4096", floor=FLOOR,
                      floor_rows=_single_key_rows(idx, bs, Hq // Hkv))
    assert_rows_close(dk, rk, BF16_REL, "dk T4096")
    assert_rows_close(dv, rv, BF16_REL, "dv T4096")


def _strided_rows(BH, T, step, offset, extra):
    """Flat rows (bh * T + i) of every (b, h) at positions offset, offset + step, ...
    plus the listed positions."""
    pos = np.union1d(np.arange(offset, T, step), [p for p in extra if 0 <= p < T])
    return (np.arange(BH)[:, None] * T + pos[None, :]).reshape(-1).astype(np.int64)


def test_nsa_bwd_T32768_G16_dense_slice(gpu):
    """B=1 Hq=64 Hkv=4 T=32768 D=128 bs=64 S=16: every element of dq on every head at every
    8th query position (and 1, 63, T-1), and of dk, dv on every kv head at every 8th key
    position (and 0, 63, 64, T-1), against the oracle in one call (the softmax statistics
    of all 2,097,152 query rows, then 262,336 dq rows and 16,400 dk/dv rows; about a
    minute on 16 threads)."""
    c = inputs.CONFIGS["nsa_bf16_T32768_G16"]
    B, Hq, Hkv, T, D, bs, S = c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["block_size"], c["S"]
    print("nsa_bwd T32768: inputs", flush=True)
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=0)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=0)
    do = _dout((B, Hq, T, D), seed=1)
    dq, dk, dv = _run(q, k, v, idx, bs, do, gpu)
    qrows = _strided_rows(B * Hq, T, 8, 0, (1, 63, T - 1))
    krows = _strided_rows(B * Hkv, T, 8, 3, (0, 63, 64, T - 1))
    print(f"nsa_bwd T32768: oracle on {qrows.size} dq rows, {krows.size} dk/dv rows", flush=True)
    rq, rk, rv = oracle.nsa_bwd_ref(q, k, v, idx, bs, do, qrows=qrows, krows=krows)
    one = _single_key_rows(idx, bs, Hq // Hkv).reshape(-1)[qrows]
    assert_rows_close(dq.reshape(-1, D)[qrows], rq, BF16_REL, "dq T32768",
                      floor=FLOOR, floor_rows=one)
    assert_rows_close(dk.reshape(-1, D)[krows], rk, BF16_REL, "dk T32768")
    assert_rows_close(dv.reshape(-1, D)[krows], rv, BF16_REL, "dv T32768")


def test_nsa_bwd_long_T131072_G16_sampled_rows(gpu):
    """B=1 Hq=16 Hkv=1 T=131072 D=128 bs=64 S=16 (2048 blocks): dq on every head at the
    first four query positions, one in 512 and the last 64; dk and dv at one key position
    in 64 (and 0, 63, 64, T-1), against the oracle in one call."""
    B, Hq, Hkv, T, D, bs, S = 1, 16, 1, 131072, 128, 64, 16
    print("nsa_bwd T131072: inputs", flush=True)
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=22)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=22)
    do = _dout((B, Hq, T, D), seed=23)
    dq, dk, dv = _run(q, k, v, idx, bs, do, gpu)
    qrows = _strided_rows(B * Hq, T, 512, 7, (0, 1, 2, 3) + tuple(range(T - 64, T)))
    krows = _strided_rows(B * Hkv, T, 64, 3, (0, 63, 64, T - 1))
    print(f"nsa_bwd T131072: oracle on {qrows.size} dq rows, {krows.size} dk/dv rows", flush=True)
    rq, rk, rv = oracle.nsa_bwd_ref(q, k, v, idx, bs, do, qrows=qrows, krows=krows)
    one = _single_key_rows(idx, bs, Hq // Hkv).reshape(-1)[qrows]
    assert_rows_close(dq.reshape(-1, D)[qrows], rq, BF16_REL, "dq T131072",
                      floor=FLOOR, floor_rows=one)
    assert_rows_close(dk.reshape(-1, D)[krows], rk, BF16_REL, "dk T131072")
    assert_rows_close(dv.reshape(-1, D)[krows], rv, BF16_REL, "dv T131072")
