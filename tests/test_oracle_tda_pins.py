"""Pins for the Threshold Differential Attention oracle (TDA page
"triton_threshold_attention.py", `differential_threshold_rela_triton`), checked
on the CPU: a hand-worked example, a closed form with a negative threshold,
the reductions the definition fixes (lambda = 0, identical paths, the clamp of
lambda), invariance of the normalised form under positive row scaling,
linearity, and a brute-force matrix evaluation on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from causal_attention_tiled_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f32(a):
    return torch.tensor(np.asarray(a, dtype=np.float32))


def _five(B, H, T, D, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(B, H, T, D, generator=g, dtype=torch.float32) for _ in range(5)]


@pytest.mark.parametrize("mode", ["normalize_bf16", "normalize_f32", "raw", "raw_bf16"])
def test_tda_hand_example(mode):
    """3-token example worked by hand (tests/golden/tda_hand_T3_D2.json).  With bf16
    inputs the normalised rows are rounded to bf16 (exact fractions in the fixture);
    with fp32 inputs to fp32, which moves the decimal hand values by ~1e-7."""
    with open(os.path.join(GOLDEN, "tda_hand_T3_D2.json")) as f:
        g = json.load(f)
    t = (lambda a: _f32(a).to(torch.bfloat16)) if mode.endswith("bf16") else _f32
    q1, k1, q2, k2, v = (t(g[n])[None, None] for n in ("q1", "k1", "q2", "k2", "v"))
    out = oracle.tda_ref(q1, q2, k1, k2, v, g["beta"], g["lambda"], g["p"],
                         normalize=mode.startswith("normalize"))[0, 0]
    key = "raw" if mode.startswith("raw") else mode
    rtol = 1e-6 if mode == "normalize_f32" else 1e-15
    np.testing.assert_allclose(out, np.asarray(g["expected"][key]), rtol=rtol, atol=rtol)


@pytest.mark.parametrize("beta,lam,p", [(-0.7, 0.3, 2.0), (-1.5, 1.0, 1.0), (-0.2, 0.75, 1.5)])
def test_tda_closed_form_negative_threshold(beta, lam, p):
    """Path 1 has cosine 1 for every pair, path 2 cosine 0; with beta < 0 the
    threshold tau_i = beta*sqrt(2 ln(i+1)/D) is <= 0, so path 1 weighs every key by
    (1 - tau_i)^p and path 2 by (-tau_i)^p (0 at i = 0), and
    out_i = ((1 - tau_i)^p - lambda (-tau_i)^p) * sum_{j<=i} v_j."""
    T, D = 7, 4
    g = torch.Generator().manual_seed(3)
    e0 = torch.zeros(T, D); e0[:, 0] = 1.0
    e1 = torch.zeros(T, D); e1[:, 1] = 1.0
    scale = torch.rand(T, 1, generator=g) * 3 + 0.5          # normalisation removes it
    q1, k1 = (e0 * scale)[None, None], (e0 * scale.flip(0))[None, None]
    q2, k2 = (e0 * scale)[None, None], (e1 * scale)[None, None]
    v = torch.randn(1, 1, T, D, generator=g)
    out = oracle.tda_ref(q1, q2, k1, k2, v, beta, lam, p, normalize=True)[0, 0]
    csum = np.cumsum(v[0, 0].double().numpy(), axis=0)
    for i in range(T):
        tau = beta * math.sqrt(2.0 * math.log(i + 1) / D)
        w = (1.0 - tau) ** p - lam * ((-tau) ** p if tau < 0 else 0.0)
        np.testing.assert_allclose(out[i], w * csum[i], rtol=1e-12, atol=1e-12)


def test_tda_lambda_zero_is_tra_on_path_one():
    q1, q2, k1, k2, v = _five(2, 2, 19, 8, seed=5)
    for norm in (False, True):
        a = oracle.tda_ref(q1, q2, k1, k2, v, 0.4, 0.0, 2.0, normalize=norm)
        if norm:
            q1n = torch.nn.functional.normalize(q1.double(), dim=-1).float()
            k1n = torch.nn.functional.normalize(k1.double(), dim=-1).float()
            b = oracle.tra_ref(q1n, k1n, v, 0.4, 2.0)
            assert np.array_equal(a, b)        # the normalised rows rounded to fp32 both ways
        else:
            assert np.array_equal(a, oracle.tra_ref(q1, k1, v, 0.4, 2.0))


def test_tda_identical_paths_cancel_at_lambda_one():
    q1, _, k1, _, v = _five(1, 3, 17, 8, seed=6)
    out = oracle.tda_ref(q1, q1, k1, k1, v, 0.1, 1.0, 2.0, normalize=True)
    assert np.all(out == 0.0)


def test_tda_lambda_is_clamped_to_unit_interval():
    q1, q2, k1, k2, v = _five(1, 2, 13, 8, seed=7)
    f = lambda lam: oracle.tda_ref(q1, q2, k1, k2, v, 0.05, lam, 2.0, normalize=True)
    assert np.array_equal(f(3.0), f(1.0))
    assert np.array_equal(f(-2.0), f(0.0))
    assert not np.array_equal(f(0.5), f(0.0))


def test_tda_affine_in_lambda():
    """out(lambda) = out1 - lambda*out2 is affine: out(0.3) = 0.7 out(0) + 0.3 out(1)."""
    q1, q2, k1, k2, v = _five(1, 2, 23, 8, seed=8)
    f = lambda lam: oracle.tda_ref(q1, q2, k1, k2, v, 0.05, lam, 2.0, normalize=True)
    np.testing.assert_allclose(f(0.3), 0.7 * f(0.0) + 0.3 * f(1.0), rtol=1e-12, atol=1e-12)


def test_tda_normalised_form_ignores_positive_row_scaling():
    q1, q2, k1, k2, v = _five(1, 2, 21, 8, seed=9)
    g = torch.Generator().manual_seed(10)
    # powers of two, so the scaled inputs are exact in fp32
    sc = [2.0 ** torch.randint(-3, 4, (1, 2, 21, 1), generator=g).float() for _ in range(4)]
    a = oracle.tda_ref(q1, q2, k1, k2, v, 0.05, 0.6, 2.0, normalize=True)
    b = oracle.tda_ref(q1 * sc[0], q2 * sc[1], k1 * sc[2], k2 * sc[3], v, 0.05, 0.6, 2.0,
                       normalize=True)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-12)
    # without normalisation the scaling matters
    c = oracle.tda_ref(q1 * sc[0], q2, k1, k2, v, 0.05, 0.6, 2.0, normalize=False)
    assert not np.allclose(c, oracle.tda_ref(q1, q2, k1, k2, v, 0.05, 0.6, 2.0, normalize=False))


def test_tda_linear_in_v():
    q1, q2, k1, k2, _ = _five(1, 2, 15, 8, seed=11)
    g = torch.Generator().manual_seed(12)
    # small dyadic values, so 2*v - v2 is exact in fp32
    v, v2 = (torch.randint(-64, 65, (1, 2, 15, 8), generator=g).float() / 16 for _ in range(2))
    f = lambda vv: oracle.tda_ref(q1, q2, k1, k2, vv, 0.05, 0.4, 2.0, normalize=True)
    np.testing.assert_allclose(f(2 * v - v2), 2 * f(v) - f(v2), rtol=1e-10, atol=1e-10)


def test_tda_zero_query_rows_contribute_nothing():
    """A zero row normalises to zero (the 1e-12 floor): its cosines are 0, below every
    non-negative threshold except at i = 0, where tau = 0 and 0^p = 0."""
    q1, q2, k1, k2, v = _five(1, 1, 9, 8, seed=13)
    q1[0, 0, 4] = 0.0
    q2[0, 0, 4] = 0.0
    out = oracle.tda_ref(q1, q2, k1, k2, v, 0.2, 0.5, 2.0, normalize=True)
    assert np.all(out[0, 0, 4] == 0.0)


@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("p", [1.0, 2.0, 1.5])
def test_tda_brute_force_matrix_form(norm, p):
    """Whole-matrix evaluation with numpy: scores as Q K^T, a lower-triangular mask,
    thresholds per row, the two weight matrices combined before the product with V."""
    B, H, T, D = 1, 2, 12, 8
    q1, q2, k1, k2, v = _five(B, H, T, D, seed=14)
    beta, lam = 0.05 if norm else 0.3, 0.35
    got = oracle.tda_ref(q1, q2, k1, k2, v, beta, lam, p, normalize=norm)
    def nrm(x):
        x = x.double().numpy()
        if not norm:
            return x
        # normalised rows go back to the inputs' dtype (fp32 here; numpy rounds to nearest even)
        y = x / np.maximum(np.linalg.norm(x, axis=-1, keepdims=True), 1e-12)
        return y.astype(np.float32).astype(np.float64)
    Q1, Q2, K1, K2 = nrm(q1), nrm(q2), nrm(k1), nrm(k2)
    V = v.double().numpy()
    tau = beta * np.sqrt(2.0 * np.log(np.arange(T) + 1.0) / D)[:, None]
    mask = np.tril(np.ones((T, T), dtype=bool))
    for b in range(B):
        for h in range(H):
            W1 = np.where(mask, np.maximum(Q1[b, h] @ K1[b, h].T - tau, 0.0) ** p, 0.0)
            W2 = np.where(mask, np.maximum(Q2[b, h] @ K2[b, h].T - tau, 0.0) ** p, 0.0)
            np.testing.assert_allclose(got[b, h], (W1 - lam * W2) @ V[b, h], rtol=1e-10, atol=1e-10)


def test_tda_rows_subset_matches_full():
    q1, q2, k1, k2, v = _five(2, 2, 11, 8, seed=15)
    full = oracle.tda_ref(q1, q2, k1, k2, v, 0.1, 0.5, 2.0).reshape(-1, 8)
    rows = np.array([0, 5, 21, 43, 10])
    part = oracle.tda_ref(q1, q2, k1, k2, v, 0.1, 0.5, 2.0, rows=rows)
    assert np.array_equal(part, full[rows])


def test_tda_normalised_bf16_rows_match_an_independent_rounding():
    """The oracle's bf16 rounding of normalised rows (nearest, ties to even) against
    torch's own fp64 -> bf16 conversion, through lambda = 0 and beta = 0, p = 1 where
    the output is a plain sum of the rounded cosines times v."""
    q1, q2, k1, k2, v = inputs.tda_inputs(2, 2, 40, 64, seed=16)
    a = oracle.tda_ref(q1, q2, k1, k2, v, 0.0, 0.0, 1.0, normalize=True)
    rnd = lambda x: (x.double() / x.double().norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    b = oracle.tra_ref(rnd(q1), rnd(k1), v, 0.0, 1.0)
    assert np.array_equal(a, b)
