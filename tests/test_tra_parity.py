"""GPU parity of the Threshold Rectified Attention forward (tra_fwd, tra_fwd_f32)
against the fp64 oracle on the same seeded inputs, plus GPU-only invariants
(causality, determinism, homogeneity) that must hold bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import causal_attention_tiled_amd as cat
from causal_attention_tiled_amd import inputs

from _parity import BF16_REL, F32_REL, assert_rows_close

pytestmark = pytest.mark.gpu


def _run_bf16(q, k, v, beta, p, dev):
    out = cat.tra_fwd(q.to(dev), k.to(dev), v.to(dev), beta, p)
    torch.cuda.synchronize()
    return out.cpu()


def _run_f32(q, k, v, beta, p, dev):
    out = cat.tra_fwd_f32(q.to(dev), k.to(dev), v.to(dev), beta, p)
    torch.cuda.synchronize()
    return out.cpu()


# several workgroup tiles (256 query rows at D=128, 128 at D=64), ragged tails, single
# rows, both head dims; 128/129 and 256/257 sit on either side of a workgroup boundary
SMALL = [(1, 2, 1, 128), (1, 2, 63, 64), (2, 1, 65, 128), (1, 3, 127, 64), (1, 1, 129, 128),
         (1, 2, 128, 64), (1, 2, 129, 64), (1, 1, 256, 64), (2, 1, 257, 64), (1, 1, 256, 128),
         (1, 1, 257, 128), (2, 2, 300, 128), (1, 2, 520, 64), (1, 1, 1000, 128)]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dH%dT%dD%d" % s)
@pytest.mark.parametrize("p", [1.0, 2.0, 1.5, 1.25])
def test_tra_bf16_small(gpu, shape, p):
    B, H, T, D = shape
    print(f"tra bf16 {shape} p={p}", flush=True)
    q, k, v = inputs.tra_inputs(B, H, T, D, dtype=torch.bfloat16, seed=T + D)
    out = _run_bf16(q, k, v, 1.0, p, gpu)
    assert_rows_close(out, oracle.tra_ref(q, k, v, 1.0, p), BF16_REL, f"tra {shape} p={p}")


@pytest.mark.parametrize("beta", [0.0, -0.5, 3.0, 1e4])
@pytest.mark.parametrize("p", [1.0, 2.0, 3.0, 0.5])
def test_tra_bf16_beta_p(gpu, beta, p):
    B, H, T, D = 1, 2, 200, 128
    q, k, v = inputs.tra_inputs(B, H, T, D, dtype=torch.bfloat16, seed=11)
    out = _run_bf16(q, k, v, beta, p, gpu)
    ref = oracle.tra_ref(q, k, v, beta, p)
    assert_rows_close(out, ref, BF16_REL, f"beta={beta} p={p}")
    if beta == 1e4:
        assert torch.all(out[:, :, 1:] == 0)          # every threshold beyond reach


@pytest.mark.parametrize("shape", [(1, 2, 1, 64), (1, 2, 63, 128), (2, 1, 65, 64), (1, 2, 200, 128)],
                         ids=lambda s: "B%dH%dT%dD%d" % s)
@pytest.mark.parametrize("p", [1.0, 2.0, 1.5, 1.25])
def test_tra_f32_small(gpu, shape, p):
    B, H, T, D = shape
    q, k, v = inputs.tra_inputs(B, H, T, D, dtype=torch.float32, seed=T)
    out = _run_f32(q, k, v, 0.8, p, gpu)
    assert_rows_close(out, oracle.tra_ref(q, k, v, 0.8, p), F32_REL, f"f32 {shape} p={p}")


def test_tra_config_f32_T256(gpu):
    """fp32, B=1 H=2 T=256 D=64, beta=1, p=2, seed 0: every element."""
    c = inputs.CONFIGS["tra_f32_T256"]
    q, k, v = inputs.tra_inputs(c["B"], c["H"], c["T"], c["D"], dtype=torch.float32, seed=0)
    out = _run_f32(q, k, v, c["beta"], 2.0, gpu)
    assert_rows_close(out, oracle.tra_ref(q, k, v, c["beta"], 2.0), F32_REL, "f32 T256")


@pytest.mark.parametrize("p", [2.0, 1.5])
def test_tra_f32_T1024_D128(gpu, p):
    """fp32, B=1 H=2 T=1024 D=128, beta=1: 16 key tiles per row block, every element."""
    q, k, v = inputs.tra_inputs(1, 2, 1024, 128, dtype=torch.float32, seed=3)
    out = _run_f32(q, k, v, 1.0, p, gpu)
    assert_rows_close(out, oracle.tra_ref(q, k, v, 1.0, p), F32_REL, f"f32 T1024 D128 p={p}")


@pytest.mark.parametrize("p", [1.0, 2.0, 1.5, 1.25])
def test_tra_config_bf16_T2048_D64(gpu, p):
    """bf16, B=4 H=16 T=2048 D=64, beta=1, p in {1, 2, 1.5}: every element."""
    c = inputs.CONFIGS["tra_bf16_T2048_D64"]
    print(f"tra config T2048 D64 p={p}: inputs", flush=True)
    q, k, v = inputs.tra_inputs(c["B"], c["H"], c["T"], c["D"], dtype=torch.bfloat16, seed=0)
    out = _run_bf16(q, k, v, c["beta"], p, gpu)
    print("  oracle (all rows)", flush=True)
    ref = oracle.tra_ref(q, k, v, c["beta"], p)
    assert_rows_close(out, ref, BF16_REL, f"T2048 p={p}")


def _long_rows(T):
    """Rows of one head at a long sequence: the first four, one in 512, and the last 64."""
    return np.unique(np.concatenate([np.arange(4), np.arange(7, T, 512), np.arange(T - 64, T)]))


@pytest.mark.parametrize("D", [128, 64])
def test_tra_long_T65536_sampled_rows(gpu, D):
    """bf16, B=1 H=1 T=65536 (1024 key tiles): the first rows, one row in 512 and the last
    64 rows against the oracle."""
    T = 65536
    print(f"tra T65536 D{D}", flush=True)
    q, k, v = inputs.tra_inputs(1, 1, T, D, seed=11)
    out = _run_bf16(q, k, v, 1.0, 2.0, gpu).reshape(-1, D)
    rows = _long_rows(T)
    ref = oracle.tra_ref(q, k, v, 1.0, 2.0, rows=rows)
    assert_rows_close(out[rows], ref, BF16_REL, f"T65536 D{D}")


@pytest.fixture(scope="module")
def big_tra():
    c = inputs.CONFIGS["tra_bf16_T8192_D128"]
    q, k, v = inputs.tra_inputs(c["B"], c["H"], c["T"], c["D"], dtype=torch.bfloat16, seed=0)
    return c, q, k, v


def test_tra_config_bf16_T8192_D128_all_rows(gpu, big_tra):
    """bf16, B=2 H=32 T=8192 D=128, beta=1, p=2 (the benchmarked launch): every
    element of the GPU output against the oracle's full output."""
    c, q, k, v = big_tra
    print("tra config T8192: gpu", flush=True)
    out = _run_bf16(q, k, v, c["beta"], 2.0, gpu)
    print("tra config T8192: oracle (all 524288 rows)", flush=True)
    ref = oracle.tra_ref(q, k, v, c["beta"], 2.0)
    print("tra config T8192: compare", flush=True)
    assert_rows_close(out, ref, BF16_REL, "T8192 all rows")


@pytest.mark.parametrize("D", [64, 128])
def test_tra_causality_bitexact(gpu, D):
    """Changing K/V at positions > c must not change any output row <= c."""
    B, H, T = 1, 2, 700
    q, k, v = inputs.tra_inputs(B, H, T, D, dtype=torch.bfloat16, seed=3)
    a = _run_bf16(q, k, v, 1.0, 2.0, gpu)
    for c in (0, 63, 64, 127, 128, 200, 255, 511):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, c + 1:] = torch.randn_like(k2[:, :, c + 1:].float()).to(k.dtype) * 3
        v2[:, :, c + 1:] = torch.randn_like(v2[:, :, c + 1:].float()).to(v.dtype) * 3
        b = _run_bf16(q, k2, v2, 1.0, 2.0, gpu)
        assert torch.equal(a[:, :, :c + 1], b[:, :, :c + 1]), f"leak past position {c}"


def test_tra_deterministic(gpu):
    q, k, v = inputs.tra_inputs(2, 4, 1024, 128, dtype=torch.bfloat16, seed=4)
    a = _run_bf16(q, k, v, 1.0, 1.5, gpu)
    b = _run_bf16(q, k, v, 1.0, 1.5, gpu)
    assert torch.equal(a, b)


@pytest.mark.parametrize("p,factor", [(1.0, 2.0), (2.0, 4.0)])
def test_tra_homogeneity_bitexact(gpu, p, factor):
    """beta = 0: tra(2Q) = 2^p tra(Q) exactly (scaling by 2 commutes with every rounding)."""
    q, k, v = inputs.tra_inputs(1, 2, 300, 64, dtype=torch.bfloat16, seed=5)
    a = _run_bf16(q, k, v, 0.0, p, gpu)
    b = _run_bf16(q * 2, k, v, 0.0, p, gpu)
    assert torch.equal(b, (a.float() * factor).to(torch.bfloat16))


def test_tra_general_p_path_matches_fast_path(gpu):
    """p = the next fp32 above 2 takes the exp2/log2 path; it must stay within
    tolerance of the exact x*x path."""
    q, k, v = inputs.tra_inputs(1, 2, 256, 128, dtype=torch.bfloat16, seed=6)
    p_next = float(np.nextafter(np.float32(2.0), np.float32(3.0)))
    a = _run_bf16(q, k, v, 1.0, 2.0, gpu)
    b = _run_bf16(q, k, v, 1.0, p_next, gpu)
    assert_rows_close(b, a.double().numpy(), BF16_REL, "general-p vs p=2")


@pytest.mark.parametrize("D", [128, 64])
def test_tra_general_p_path_matches_three_halves_path(gpu, D):
    """p = the next fp32 above 1.5 takes the exp2/log2 path, p = 1.5 the r*sqrt(r) one:
    within tolerance of each other, bf16 and fp32."""
    p_next = float(np.nextafter(np.float32(1.5), np.float32(2.0)))
    q, k, v = inputs.tra_inputs(1, 2, 300, D, dtype=torch.bfloat16, seed=8)
    a = _run_bf16(q, k, v, 1.0, 1.5, gpu)
    b = _run_bf16(q, k, v, 1.0, p_next, gpu)
    assert_rows_close(b, a.double().numpy(), BF16_REL, "general-p vs p=1.5, bf16")
    q, k, v = inputs.tra_inputs(1, 2, 300, D, dtype=torch.float32, seed=8)
    a = _run_f32(q, k, v, 1.0, 1.5, gpu)
    b = _run_f32(q, k, v, 1.0, p_next, gpu)
    assert_rows_close(b, a.double().numpy(), F32_REL, "general-p vs p=1.5, fp32")


def test_tra_empty_is_noop(gpu):
    q = torch.zeros(0, 2, 16, 64, dtype=torch.bfloat16, device=gpu)
    out = cat.tra_fwd(q, q, q, 1.0, 2.0)
    assert out.shape == q.shape
