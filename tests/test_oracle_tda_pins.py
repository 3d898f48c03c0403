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
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from causal_attention_tiled_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f32(a):
    return torch.tensor(np.asarray(a, dtype=np.float32))


def _normalize_f32(x):
    """Rows of an fp32 tensor normalised under the page's reading, computed with numpy:
    the 2-norm rounded to fp32 (at least 1e-12), then an fp32 division (correctly
    rounded), as torch.nn.functional.normalize does on an fp32 tensor up to the
    rounding of its own accumulation."""
    x = x.numpy().astype(np.float32)
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True)).astype(np.float32)
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float64)


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
            q1n = torch.tensor(_normalize_f32(q1), dtype=torch.float32)
            k1n = torch.tensor(_normalize_f32(k1), dtype=torch.float32)
            b = oracle.tra_ref(q1n, k1n, v, 0.4, 2.0)
            assert np.array_equal(a, b)        # the same fp32 normalised rows both ways
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
        return _normalize_f32(x) if norm else x.double().numpy()
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


def _bf16_rne(x):
    """Exact round-to-nearest-even of a Fraction to bf16 (8 significant bits)."""
    if x == 0:
        return Fraction(0)
    sgn, a = (-1 if x < 0 else 1), abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = a / Fraction(2) ** (e - 7)
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sgn * n * Fraction(2) ** (e - 7)


def _bf16_exact_normalise(row):
    """Exact rational evaluation of one bf16 row's normalisation: the bf16 value
    nearest to sqrt(sum x^2), found by comparing the squares of the bf16 midpoints
    with the exact sum, then each x / norm rounded to bf16."""
    xs = [Fraction(float(x)) for x in row]
    ss = sum(x * x for x in xs)
    if ss == 0:
        return [0.0] * len(xs)
    c = _bf16_rne(Fraction(math.sqrt(float(ss))))
    while True:                      # move c until sqrt(ss) lies within its rounding interval
        e = c.numerator.bit_length() - c.denominator.bit_length()
        while Fraction(2) ** e > c:
            e -= 1
        ulp = Fraction(2) ** (e - 7)
        below = ulp / 2 if c > Fraction(2) ** e else ulp / 4   # a binade start has a finer gap below
        lo, hi = c - below, c + ulp / 2
        if lo * lo > ss or (lo * lo == ss and (c / ulp) % 2 == 1):
            c -= 2 * below
        elif hi * hi < ss or (hi * hi == ss and (c / ulp) % 2 == 1):
            c += ulp
        else:
            break
    return [float(_bf16_rne(x / c)) for x in xs]


@pytest.mark.parametrize("D", [64, 128])
def test_tda_normalised_bf16_rows_match_torch_normalize(D):
    """The oracle's normalised bf16 rows against torch.nn.functional.normalize on the
    same bf16 tensors, bit for bit.  torch sums the squares in fp32, so where the exact
    norm lies within 2^-20 (relative) of a bf16 rounding midpoint its bf16 norm may fall
    on the other side; those rows (about one in 10^3) are checked instead against an exact
    rational evaluation of the same definition."""
    rows_checked = ambiguous = 0
    for seed in range(3):
        for x in inputs.tda_inputs(1, 4, 2048, D, seed=100 + seed)[:4]:
            got = oracle.l2norm_ref(x).reshape(-1, D)
            want = torch.nn.functional.normalize(x, dim=-1).double().numpy().reshape(-1, D)
            xd = x.double().reshape(-1, D).numpy()
            nrm = np.sqrt(np.sum(xd * xd, axis=1))
            ulp = 2.0 ** (np.floor(np.log2(nrm)) - 7)
            near_tie = np.abs(np.mod(nrm / ulp, 1.0) - 0.5) * ulp / nrm < 2.0 ** -20
            assert np.array_equal(got[~near_tie], want[~near_tie])
            for r in np.nonzero(near_tie)[0]:
                assert got[r].tolist() == _bf16_exact_normalise(x.reshape(-1, D)[r])
            rows_checked += got.shape[0]
            ambiguous += int(near_tie.sum())
    assert ambiguous <= rows_checked // 400


def test_tda_normalised_bf16_rows_hand_values():
    """The rows of tests/golden/tda_hand_norm_rounding_T2_D2.json, worked by hand, and
    the same rows through torch.nn.functional.normalize in bf16."""
    with open(os.path.join(GOLDEN, "tda_hand_norm_rounding_T2_D2.json")) as f:
        g = json.load(f)
    for name in ("q1", "k1"):
        x = _f32(g[name]).to(torch.bfloat16)
        want = np.asarray(g["normalised_rows"][name])
        assert np.array_equal(oracle.l2norm_ref(x), want)
        assert np.array_equal(torch.nn.functional.normalize(x, dim=-1).double().numpy(), want)
        assert [_bf16_exact_normalise(r) for r in x] == want.tolist()


def test_tda_hand_example_norm_rounding():
    """2-token bf16 example whose row norms are not bf16 values (worked by hand in
    tests/golden/tda_hand_norm_rounding_T2_D2.json): rounding the norm before the
    divide moves the normalised rows, and the output, away from the exact-quotient
    rounding."""
    with open(os.path.join(GOLDEN, "tda_hand_norm_rounding_T2_D2.json")) as f:
        g = json.load(f)
    q1, k1, q2, k2, v = (_f32(g[n]).to(torch.bfloat16)[None, None]
                         for n in ("q1", "k1", "q2", "k2", "v"))
    out = oracle.tda_ref(q1, q2, k1, k2, v, g["beta"], g["lambda"], g["p"], normalize=True)
    assert np.array_equal(out[0, 0], np.asarray(g["expected"]))


def test_tda_normalised_output_equals_tra_on_torch_normalised_rows():
    """lambda = 0: the normalised differential forward is the rectified forward of path 1
    on torch's bf16-normalised q1 and k1 rows (inputs chosen with no near-tie norm)."""
    q1, q2, k1, k2, v = inputs.tda_inputs(1, 2, 150, 64, seed=17)
    a = oracle.tda_ref(q1, q2, k1, k2, v, 0.05, 0.0, 2.0, normalize=True)
    nq, nk = (torch.nn.functional.normalize(x, dim=-1) for x in (q1, k1))
    assert np.array_equal(oracle.l2norm_ref(q1), nq.double().numpy())
    assert np.array_equal(oracle.l2norm_ref(k1), nk.double().numpy())
    assert np.array_equal(a, oracle.tra_ref(nq, nk, v, 0.05, 2.0))
