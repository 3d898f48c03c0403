"""GPU parity of the Threshold Differential Attention forward (tda_fwd) against
the fp64 oracle on the same seeded inputs, plus GPU-only identities that must
hold bit for bit (lambda = 0 is the rectified forward of path 1, identical paths
cancel, causality, determinism)."""
import numpy as np
import pytest
import torch

import oracle
import causal_attention_tiled_amd as cat
from causal_attention_tiled_amd import inputs

from _parity import BF16_REL, assert_rows_close

pytestmark = pytest.mark.gpu


def _run(t5, beta, lam, p, normalize, dev):
    out = cat.tda_fwd(*(t.to(dev) for t in t5), beta, lam, p, normalize=normalize)
    torch.cuda.synchronize()
    return out.cpu()


SMALL = [(1, 2, 1, 128), (1, 2, 63, 64), (2, 1, 65, 128), (1, 1, 129, 64), (1, 2, 300, 128),
         (2, 1, 520, 64), (1, 1, 777, 128)]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dH%dT%dD%d" % s)
@pytest.mark.parametrize("normalize", [True, False], ids=["norm", "raw"])
@pytest.mark.parametrize("p", [1.0, 2.0, 1.5, 1.25])
def test_tda_small(gpu, shape, normalize, p):
    B, H, T, D = shape
    print(f"tda {shape} normalize={normalize} p={p}", flush=True)
    t5 = inputs.tda_inputs(B, H, T, D, seed=T + D)
    beta = 0.05 if normalize else 0.5
    out = _run(t5, beta, 0.6, p, normalize, gpu)
    ref = oracle.tda_ref(*t5, beta, 0.6, p, normalize=normalize)
    assert_rows_close(out, ref, BF16_REL, f"tda {shape} norm={normalize} p={p}")


@pytest.mark.parametrize("lam", [0.0, 0.25, 1.0, 3.0, -1.0])
@pytest.mark.parametrize("beta", [0.0, -0.1, 0.1])
def test_tda_lambda_beta(gpu, lam, beta):
    B, H, T, D = 1, 2, 200, 128
    t5 = inputs.tda_inputs(B, H, T, D, seed=21)
    out = _run(t5, beta, lam, 2.0, True, gpu)
    assert_rows_close(out, oracle.tda_ref(*t5, beta, lam, 2.0, normalize=True), BF16_REL,
                      f"lam={lam} beta={beta}")


def test_tda_config_T8192_D128_all_rows(gpu):
    """B=2 H=32 T=8192 D=128, normalised, beta = D^-1/2, lambda = 0.5, p = 2 (the
    benchmarked launch): every element of the output against the oracle."""
    c = inputs.CONFIGS["tda_bf16_T8192_D128"]
    print("tda config T8192: inputs", flush=True)
    t5 = inputs.tda_inputs(c["B"], c["H"], c["T"], c["D"], seed=0)
    out = _run(t5, c["beta"], c["lam"], 2.0, c["normalize"], gpu)
    print("tda config T8192: oracle on all 524,288 rows", flush=True)
    ref = oracle.tda_ref(*t5, c["beta"], c["lam"], 2.0, normalize=c["normalize"])
    assert_rows_close(out, ref, BF16_REL, "tda T8192")


def test_tda_long_T32768_sampled_rows(gpu):
    """Normalised, B=1 H=1 T=32768 D=128, beta=D^-1/2, lambda=0.5, p=2: the first rows, one
    row in 512 and the last 64 rows against the oracle."""
    T, D = 32768, 128
    print("tda T32768", flush=True)
    t5 = inputs.tda_inputs(1, 1, T, D, seed=14)
    out = _run(t5, D ** -0.5, 0.5, 2.0, True, gpu).reshape(-1, D)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(7, T, 512), np.arange(T - 64, T)]))
    ref = oracle.tda_ref(*t5, D ** -0.5, 0.5, 2.0, normalize=True, rows=rows)
    assert_rows_close(out[rows], ref, BF16_REL, "tda T32768")


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("p", [1.0, 2.0, 1.5, 1.25])
def test_tda_lambda_zero_matches_tra(gpu, p, D):
    """lambda = 0, no normalisation: the output is the rectified forward of path 1, bit
    for bit (both kernels start the scores at -tau, accumulate the same products in the
    same order, and the second path's weight enters as -0 * w2 + w1 = w1)."""
    t5 = inputs.tda_inputs(1, 2, 333, D, seed=22)
    a = _run(t5, 0.7, 0.0, p, False, gpu)
    q1, _, k1, _, v = (t.to(gpu) for t in t5)
    b = cat.tra_fwd(q1, k1, v, 0.7, p).cpu()
    assert torch.equal(a, b), f"lambda 0 vs tra D={D} p={p}"


def test_tda_identical_paths_cancel_bitexact(gpu):
    q1, _, k1, _, v = inputs.tda_inputs(1, 2, 300, 64, seed=23)
    for norm in (True, False):
        out = _run((q1, q1, k1, k1, v), 0.05 if norm else 0.5, 1.0, 2.0, norm, gpu)
        assert torch.all(out == 0)


def test_tda_causality_bitexact(gpu):
    t5 = list(inputs.tda_inputs(1, 2, 600, 128, seed=24))
    a = _run(t5, 0.05, 0.5, 2.0, True, gpu)
    for c in (0, 63, 64, 255, 400):
        t = [x.clone() for x in t5]
        for idx in (2, 3, 4):                       # k1, k2, v after position c
            t[idx][:, :, c + 1:] = torch.randn_like(t[idx][:, :, c + 1:].float()).to(torch.bfloat16)
        b = _run(t, 0.05, 0.5, 2.0, True, gpu)
        assert torch.equal(a[:, :, :c + 1], b[:, :, :c + 1]), f"leak past position {c}"


def test_tda_deterministic_and_workspace_reuse(gpu):
    t5 = [x.to(gpu) for x in inputs.tda_inputs(2, 2, 700, 128, seed=25)]
    ws = torch.empty(cat.tda_workspace_bytes(2, 2, 700, 128), dtype=torch.uint8, device=gpu)
    a = cat.tda_fwd(*t5, 0.05, 0.5, 1.5, workspace=ws)
    b = cat.tda_fwd(*t5, 0.05, 0.5, 1.5, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_tda_empty_is_noop(gpu):
    z = torch.empty(1, 2, 0, 128, dtype=torch.bfloat16, device=gpu)
    out = cat.tda_fwd(z, z, z, z, z, 0.1, 0.5, 2.0)
    assert out.shape == z.shape
