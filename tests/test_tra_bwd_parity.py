"""GPU parity of the Threshold Rectified Attention backward (tra_bwd) against the
fp64 oracle on the same seeded inputs, plus GPU-only properties that must hold bit
for bit (determinism, causal dependency structure)."""
import numpy as np
import pytest
import torch

import oracle
import causal_attention_tiled_amd as cat
from causal_attention_tiled_amd import inputs

from _parity import BF16_REL, assert_rows_close

pytestmark = pytest.mark.gpu


def _dout(B, H, T, D, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(B, H, T, D, generator=g).to(torch.bfloat16)


def _run(q, k, v, do, beta, p, dev):
    g = cat.tra_bwd(q.to(dev), k.to(dev), v.to(dev), do.to(dev), beta, p)
    torch.cuda.synchronize()
    return [x.cpu() for x in g]


# At D = 128 the dk/dv kernel takes 256 keys per workgroup (64 per wave): T = 256, 257, 511
# and 1000 give an exact workgroup, one holding a single key, waves whose keys all lie
# past T, and a ragged last workgroup.
SMALL = [(1, 2, 1, 128), (1, 2, 63, 64), (2, 1, 65, 128), (1, 1, 129, 64), (1, 2, 300, 128),
         (2, 1, 520, 64), (1, 1, 777, 128), (1, 1, 256, 128), (1, 2, 257, 128), (2, 1, 511, 128),
         (1, 1, 1000, 128)]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dH%dT%dD%d" % s)
@pytest.mark.parametrize("p", [1.0, 2.0, 1.5, 1.25])
def test_tra_bwd_small(gpu, shape, p):
    B, H, T, D = shape
    print(f"tra_bwd {shape} p={p}", flush=True)
    q, k, v = inputs.tra_inputs(B, H, T, D, seed=T + D)
    do = _dout(B, H, T, D, seed=T)
    got = _run(q, k, v, do, 1.0, p, gpu)
    ref = oracle.tra_bwd_ref(q, k, v, do, 1.0, p)
    for g, r, n in zip(got, ref, ("dq", "dk", "dv")):
        assert_rows_close(g, r, BF16_REL, f"{n} {shape} p={p}")


@pytest.mark.parametrize("beta,p", [(0.0, 2.0), (-0.5, 2.0), (2.0, 2.0), (0.0, 3.0), (-0.5, 3.0),
                                    (2.0, 3.0), (-0.5, 1.5)])
def test_tra_bwd_beta_p(gpu, beta, p):
    B, H, T, D = 1, 2, 200, 128
    q, k, v = inputs.tra_inputs(B, H, T, D, seed=31)
    do = _dout(B, H, T, D, seed=32)
    got = _run(q, k, v, do, beta, p, gpu)
    ref = oracle.tra_bwd_ref(q, k, v, do, beta, p)
    for g, r, n in zip(got, ref, ("dq", "dk", "dv")):
        assert_rows_close(g, r, BF16_REL, f"{n} beta={beta} p={p}")


def test_tra_bwd_p_below_one_well_conditioned(gpu):
    """p = 0.5: the weight's derivative p*x^(p-1) is unbounded as x -> 0+, so near the
    threshold a gradient follows the last bits of the fp32 score and no fixed tolerance
    holds.  With beta = -40 every pair of rows i >= 1 sits at x = q.k + 40*sqrt(2 ln(i+1)/D)
    >= 4 above it (the scores are about N(0, 1)), the well-conditioned case; row 0
    (tau_0 = 0) and key 0, which row 0 feeds, are left out."""
    B, H, T, D = 1, 2, 200, 128
    q, k, v = inputs.tra_inputs(B, H, T, D, seed=33)
    do = _dout(B, H, T, D, seed=34)
    got = _run(q, k, v, do, -40.0, 0.5, gpu)
    ref = oracle.tra_bwd_ref(q, k, v, do, -40.0, 0.5)
    for g, r, n in zip(got, ref, ("dq", "dk", "dv")):
        assert_rows_close(g[:, :, 1:], r[:, :, 1:], BF16_REL, f"{n} p=0.5")


def test_tra_bwd_T8192_D128_all_rows(gpu):
    """B=2 H=32 T=8192 D=128, beta=1, p=2 (the forward's measured shape): every element of
    dq, dk and dv against the oracle."""
    B, H, T, D = 2, 32, 8192, 128
    print("tra_bwd T8192: inputs", flush=True)
    q, k, v = inputs.tra_inputs(B, H, T, D, seed=0)
    do = _dout(B, H, T, D, seed=1)
    dq, dk, dv = _run(q, k, v, do, 1.0, 2.0, gpu)
    print("tra_bwd T8192: oracle on all 524,288 rows of each gradient", flush=True)
    rq, rk, rv = oracle.tra_bwd_ref(q, k, v, do, 1.0, 2.0)
    assert_rows_close(dq, rq, BF16_REL, "dq T8192")
    assert_rows_close(dk, rk, BF16_REL, "dk T8192")
    assert_rows_close(dv, rv, BF16_REL, "dv T8192")


@pytest.mark.parametrize("p", [2.0, 1.5])
def test_tra_bwd_T2048_D64_all_rows(gpu, p):
    """B=4 H=16 T=2048 D=64, beta=1 (the D = 64 forward's shape): every element of dq, dk
    and dv against the oracle."""
    B, H, T, D = 4, 16, 2048, 64
    print(f"tra_bwd T2048 D64 p={p}", flush=True)
    q, k, v = inputs.tra_inputs(B, H, T, D, seed=2)
    do = _dout(B, H, T, D, seed=3)
    dq, dk, dv = _run(q, k, v, do, 1.0, p, gpu)
    rq, rk, rv = oracle.tra_bwd_ref(q, k, v, do, 1.0, p)
    assert_rows_close(dq, rq, BF16_REL, f"dq T2048 D64 p={p}")
    assert_rows_close(dk, rk, BF16_REL, f"dk T2048 D64 p={p}")
    assert_rows_close(dv, rv, BF16_REL, f"dv T2048 D64 p={p}")


@pytest.mark.parametrize("D", [128, 64])
def test_tra_bwd_long_T65536_sampled_rows(gpu, D):
    """B=1 H=1 T=65536 (256 key workgroups at D=128, 512 at D=64): dq on the first rows,
    one row in 512 and the last 64, dk and dv on the same key rows, against the oracle."""
    T = 65536
    print(f"tra_bwd T65536 D{D}", flush=True)
    q, k, v = inputs.tra_inputs(1, 1, T, D, seed=12)
    do = _dout(1, 1, T, D, seed=13)
    dq, dk, dv = _run(q, k, v, do, 1.0, 2.0, gpu)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(7, T, 512), np.arange(T - 64, T)]))
    rq, rk, rv = oracle.tra_bwd_ref(q, k, v, do, 1.0, 2.0, qrows=rows, krows=rows)
    assert_rows_close(dq.reshape(-1, D)[rows], rq, BF16_REL, f"dq T65536 D{D}")
    assert_rows_close(dk.reshape(-1, D)[rows], rk, BF16_REL, f"dk T65536 D{D}")
    assert_rows_close(dv.reshape(-1, D)[rows], rv, BF16_REL, f"dv T65536 D{D}")


@pytest.mark.parametrize("D", [128, 64])
def test_tra_bwd_general_p_path_matches_three_halves_path(gpu, D):
    """p = the next fp32 above 1.5 (exp2/log2 of one shared log) against p = 1.5 (one
    square root for the weight and its derivative): within tolerance."""
    p_next = float(np.nextafter(np.float32(1.5), np.float32(2.0)))
    q, k, v = inputs.tra_inputs(1, 2, 300, D, seed=9)
    do = _dout(1, 2, 300, D, seed=10)
    a = _run(q, k, v, do, 1.0, 1.5, gpu)
    b = _run(q, k, v, do, 1.0, p_next, gpu)
    for x, y, n in zip(b, a, ("dq", "dk", "dv")):
        assert_rows_close(x, y.double().numpy(), BF16_REL, f"{n} general-p vs p=1.5")


def test_tra_bwd_deterministic(gpu):
    q, k, v = inputs.tra_inputs(2, 2, 700, 128, seed=5)
    do = _dout(2, 2, 700, 128, seed=6)
    a = _run(q, k, v, do, 1.0, 1.5, gpu)
    b = _run(q, k, v, do, 1.0, 1.5, gpu)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_tra_bwd_causal_structure_bitexact(gpu):
    """dq rows <= c ignore keys/values after c; dk, dv rows >= c ignore queries and
    output gradients before c."""
    B, H, T, D = 1, 2, 600, 128
    q, k, v = inputs.tra_inputs(B, H, T, D, seed=7)
    do = _dout(B, H, T, D, seed=8)
    a = _run(q, k, v, do, 1.0, 2.0, gpu)
    c = 300
    k2, v2 = k.clone(), v.clone()
    k2[:, :, c + 1:] = torch.randn_like(k2[:, :, c + 1:].float()).to(torch.bfloat16)
    v2[:, :, c + 1:] = torch.randn_like(v2[:, :, c + 1:].float()).to(torch.bfloat16)
    b = _run(q, k2, v2, do, 1.0, 2.0, gpu)
    assert torch.equal(a[0][:, :, :c + 1], b[0][:, :, :c + 1])
    q2, do2 = q.clone(), do.clone()
    q2[:, :, :c] = torch.randn_like(q2[:, :, :c].float()).to(torch.bfloat16)
    do2[:, :, :c] = torch.randn_like(do2[:, :, :c].float()).to(torch.bfloat16)
    b = _run(q2, k, v, do2, 1.0, 2.0, gpu)
    assert torch.equal(a[1][:, :, c:], b[1][:, :, c:])
    assert torch.equal(a[2][:, :, c:], b[2][:, :, c:])


def test_tra_bwd_empty_is_noop(gpu):
    z = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device=gpu)
    dq, dk, dv = cat.tra_bwd(z, z, z, z, 1.0, 2.0)
    assert dq.shape == z.shape
