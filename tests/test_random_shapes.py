"""GPU parity against the fp64 oracle on seeded random shapes and parameters: sequence
lengths that are not multiples of any tile, both head dims, powers on every path
(1, 2 and general), thresholds of either sign, GQA group sizes from 1 to 16, block
sizes 32 / 64 / 128 and block lists with padding, repeats, future and out-of-range
ids.  Every case compares every output element."""
import numpy as np
import pytest
import torch

import oracle
import causal_attention_tiled_amd as cat
from causal_attention_tiled_amd import inputs

from _parity import BF16_REL, F32_REL, assert_lse_close, assert_rows_close

pytestmark = pytest.mark.gpu

RNG_SEED = 20261203


def _cases(kind, n):
    rng = np.random.default_rng([RNG_SEED, sum(map(ord, kind))])
    return [rng.integers(0, 2**31 - 1) for _ in range(n)]


def _pick(rng, xs):
    return xs[int(rng.integers(0, len(xs)))]


@pytest.mark.parametrize("seed", _cases("tra", 20))
def test_tra_random(gpu, seed):
    rng = np.random.default_rng(seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    T, D = int(rng.integers(1, 700)), _pick(rng, [64, 128])
    p = _pick(rng, [1.0, 2.0, 1.5, 1.25, 0.5, 3.0])
    beta = float(rng.uniform(-0.5, 1.5))
    print(f"tra B{B} H{H} T{T} D{D} p{p} beta{beta:.3f}", flush=True)
    q, k, v = inputs.tra_inputs(B, H, T, D, seed=int(seed % 1000))
    out = cat.tra_fwd(q.to(gpu), k.to(gpu), v.to(gpu), beta, p)
    torch.cuda.synchronize()
    assert_rows_close(out.cpu(), oracle.tra_ref(q, k, v, beta, p), BF16_REL, f"tra seed {seed}")


@pytest.mark.parametrize("seed", _cases("tra_f32", 8))
def test_tra_f32_random(gpu, seed):
    rng = np.random.default_rng(seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    T, D = int(rng.integers(1, 320)), _pick(rng, [64, 128])
    p = _pick(rng, [1.0, 2.0, 1.5, 1.25])
    beta = float(rng.uniform(-0.5, 1.5))
    print(f"tra f32 B{B} H{H} T{T} D{D} p{p} beta{beta:.3f}", flush=True)
    q, k, v = inputs.tra_inputs(B, H, T, D, dtype=torch.float32, seed=int(seed % 1000))
    out = cat.tra_fwd_f32(q.to(gpu), k.to(gpu), v.to(gpu), beta, p)
    torch.cuda.synchronize()
    assert_rows_close(out.cpu(), oracle.tra_ref(q, k, v, beta, p), F32_REL, f"tra f32 seed {seed}")


@pytest.mark.parametrize("seed", _cases("tra_bwd", 10))
def test_tra_bwd_random(gpu, seed):
    rng = np.random.default_rng(seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    T, D = int(rng.integers(1, 420)), _pick(rng, [64, 128])
    p = _pick(rng, [1.0, 2.0, 1.5, 1.25, 3.0])
    beta = float(rng.uniform(-0.5, 1.5))
    print(f"tra_bwd B{B} H{H} T{T} D{D} p{p} beta{beta:.3f}", flush=True)
    q, k, v = inputs.tra_inputs(B, H, T, D, seed=int(seed % 1000))
    do = torch.randn(B, H, T, D, generator=torch.Generator().manual_seed(int(seed % 997)))
    do = do.to(torch.bfloat16)
    g = cat.tra_bwd(q.to(gpu), k.to(gpu), v.to(gpu), do.to(gpu), beta, p)
    torch.cuda.synchronize()
    for name, x, r in zip(("dq", "dk", "dv"), g, oracle.tra_bwd_ref(q, k, v, do, beta, p)):
        assert_rows_close(x.cpu(), r, BF16_REL, f"tra_bwd {name} seed {seed}")


@pytest.mark.parametrize("seed", _cases("tda", 10))
def test_tda_random(gpu, seed):
    rng = np.random.default_rng(seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    T, D = int(rng.integers(1, 420)), _pick(rng, [64, 128])
    p = _pick(rng, [1.0, 2.0, 1.5, 1.25])
    norm = bool(rng.integers(0, 2))
    beta = float(rng.uniform(-0.05, 0.15)) if norm else float(rng.uniform(-0.5, 1.5))
    lam = float(rng.uniform(-0.3, 1.3))
    print(f"tda B{B} H{H} T{T} D{D} p{p} beta{beta:.3f} lam{lam:.3f} norm={norm}", flush=True)
    t5 = inputs.tda_inputs(B, H, T, D, seed=int(seed % 1000))
    out = cat.tda_fwd(*(t.to(gpu) for t in t5), beta, lam, p, normalize=norm)
    torch.cuda.synchronize()
    ref = oracle.tda_ref(*t5, beta, lam, p, normalize=norm)
    assert_rows_close(out.cpu(), ref, BF16_REL, f"tda seed {seed}")


def _random_block_idx(rng, B, Hkv, T, bs, S, seed):
    """The benchmark's selection, then a random share of slots replaced by padding,
    repeats, blocks after the query and ids past the last block."""
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=seed)
    nblk = T // bs
    r = rng.random(idx.shape)
    idx = np.where(r < 0.05, -1, idx)
    idx = np.where((r >= 0.05) & (r < 0.10), np.roll(idx, 1, axis=-1), idx)
    future = np.minimum(np.arange(T)[None, None, :, None] // bs + 1, nblk)
    idx = np.where((r >= 0.10) & (r < 0.13), future, idx)
    idx = np.where((r >= 0.13) & (r < 0.15), nblk + 2, idx)
    return np.ascontiguousarray(idx.astype(np.int32))


def _nsa_case(seed, max_tokens=1536, max_g=16):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.integers(1, 4))
    G = _pick(rng, [g for g in (1, 2, 3, 4, 5, 8, 16) if g <= max_g])
    bs = _pick(rng, [32, 64, 128])
    T = bs * int(rng.integers(1, max_tokens // bs + 1))
    D = _pick(rng, [64, 128])
    S = int(rng.integers(1, 21))
    B = int(rng.integers(1, 3))
    return rng, B, Hkv * G, Hkv, T, D, bs, S


@pytest.mark.parametrize("seed", _cases("nsa", 20))
def test_nsa_random_both_forms(gpu, seed):
    rng, B, Hq, Hkv, T, D, bs, S = _nsa_case(seed)
    print(f"nsa B{B} Hq{Hq} Hkv{Hkv} T{T} D{D} bs{bs} S{S}", flush=True)
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=int(seed % 1000))
    idx = _random_block_idx(rng, B, Hkv, T, bs, S, seed=int(seed % 991))
    ro, rl = oracle.nsa_ref(q, k, v, idx, bs)
    gi = torch.from_numpy(idx).to(gpu)
    for name, fn in (("query-outer", cat.nsa_sel_fwd), ("block-outer", cat.nsa_sel_fwd_fsa)):
        o, lse = fn(q.to(gpu), k.to(gpu), v.to(gpu), gi, bs)
        torch.cuda.synchronize()
        assert_rows_close(o.cpu(), ro, BF16_REL, f"nsa {name} seed {seed}")
        assert_lse_close(lse.cpu(), rl, f"nsa {name} seed {seed}")


@pytest.mark.parametrize("seed", _cases("nsa_bwd", 8))
def test_nsa_bwd_random(gpu, seed):
    from test_nsa_bwd_parity import FLOOR, _single_key_rows
    rng, B, Hq, Hkv, T, D, bs, S = _nsa_case(seed, max_tokens=512, max_g=8)
    print(f"nsa_bwd B{B} Hq{Hq} Hkv{Hkv} T{T} D{D} bs{bs} S{S}", flush=True)
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=int(seed % 1000))
    idx = _random_block_idx(rng, B, Hkv, T, bs, S, seed=int(seed % 991))
    do = torch.randn(B, Hq, T, D, generator=torch.Generator().manual_seed(int(seed % 983)))
    do = do.to(torch.bfloat16)
    gq, gk, gv, gi = q.to(gpu), k.to(gpu), v.to(gpu), torch.from_numpy(idx).to(gpu)
    o, lse = cat.nsa_sel_fwd(gq, gk, gv, gi, bs)
    g = cat.nsa_sel_bwd(gq, gk, gv, gi, bs, o, lse, do.to(gpu))
    torch.cuda.synchronize()
    ref = oracle.nsa_bwd_ref(q, k, v, idx, bs, do)
    one = _single_key_rows(idx, bs, Hq // Hkv)
    assert_rows_close(g[0].cpu(), ref[0], BF16_REL, f"dq seed {seed}", floor=FLOOR, floor_rows=one)
    assert_rows_close(g[1].cpu(), ref[1], BF16_REL, f"dk seed {seed}")
    assert_rows_close(g[2].cpu(), ref[2], BF16_REL, f"dv seed {seed}")
