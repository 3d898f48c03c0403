"""Pins for the fp64 oracle, checked on the CPU against facts that the pages and
the mathematics fix -- hand-worked examples, closed forms, special cases that
reduce to library routines, invariants, and brute force on tiny inputs.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, index or log base, a transposed operand, a duplicate counted
twice) fails at least one of them.
"""
import itertools
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


def _rand(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32) * std


def _f64(t):
    return t.to(torch.float64).numpy()


# --------------------------------------------------------------------------
# Threshold Rectified Attention
# (TDA page "triton_threshold_attention.py": module docstring, forward kernel)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("p", ["1.0", "2.0", "3.0"])
def test_tra_hand_example(p):
    """3-token integer example worked by hand (tests/golden/tra_hand_T3_D2.json)."""
    with open(os.path.join(GOLDEN, "tra_hand_T3_D2.json")) as f:
        g = json.load(f)
    q, k, v = (_f32(g[n])[None, None] for n in ("q", "k", "v"))
    out = oracle.tra_ref(q, k, v, g["beta"], float(p))[0, 0]
    assert np.array_equal(out, np.asarray(g["expected"][p], dtype=np.float64))


@pytest.mark.parametrize("D,expect", [(2, 1.1774100225154747),   # sqrt(2 ln 2)
                                      (4, 0.8325546111576977)])  # sqrt(ln 2)
def test_tra_tau_value_at_i3(D, expect):
    """tau_3 = beta*sqrt(2 ln 4 / D) read back from the output.

    With q_i = (2,0,..), k_j = (1,0,..) every causal score is exactly 2; with
    v = 1 and p = 1, out_i = (i+1) * max(2 - tau_i, 0), so tau_i is recovered
    from the output and compared to a constant (natural log, factor 2, /D)."""
    T = 6
    q = torch.zeros(1, 1, T, D); q[..., 0] = 2.0
    k = torch.zeros(1, 1, T, D); k[..., 0] = 1.0
    v = torch.ones(1, 1, T, D)
    out = oracle.tra_ref(q, k, v, 1.0, 1.0)[0, 0]
    tau3 = 2.0 - out[3, 0] / 4.0
    assert abs(tau3 - expect) < 1e-14
    assert out[0, 0] == 2.0                      # tau_0 = 0
    taus = 2.0 - out[:, 0] / np.arange(1, T + 1)
    assert np.all(np.diff(taus) > 0)             # tau grows with position


@pytest.mark.parametrize("beta", [0.0, 1.0, 5.0, -2.0, 1e4])
@pytest.mark.parametrize("p", [1.0, 2.0, 1.5, 3.0])
def test_tra_row0_closed_form(beta, p):
    """tau_0 = 0 for every beta, so row 0 is max(q0.k0, 0)^p v0."""
    B, H, T, D = 2, 3, 5, 8
    q, k, v = _rand((B, H, T, D), 1), _rand((B, H, T, D), 2), _rand((B, H, T, D), 3)
    out = oracle.tra_ref(q, k, v, beta, p)
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    s0 = np.einsum("bhd,bhd->bh", qd[:, :, 0], kd[:, :, 0])
    w0 = np.where(s0 > 0, np.abs(s0) ** p, 0.0)
    np.testing.assert_allclose(out[:, :, 0], w0[..., None] * vd[:, :, 0], rtol=1e-13, atol=1e-15)


def test_tra_huge_beta_is_zero_after_row0():
    """beta = 1e4 puts every threshold for i >= 1 far above any score."""
    q, k, v = inputs.tra_inputs(1, 2, 40, 64, dtype=torch.float32, seed=5)
    out = oracle.tra_ref(q, k, v, 1e4, 2.0)
    assert np.all(out[:, :, 1:] == 0.0)
    assert np.any(out[:, :, 0] != 0.0)


@pytest.mark.parametrize("T,D", [(7, 4), (33, 16)])
def test_tra_beta0_p1_is_masked_matmul(T, D):
    """beta = 0, p = 1: out = (ReLU(Q K^T) masked to j <= i) V, via numpy matmul."""
    q, k, v = _rand((2, 2, T, D), 10), _rand((2, 2, T, D), 11), _rand((2, 2, T, D), 12)
    out = oracle.tra_ref(q, k, v, 0.0, 1.0)
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    s = qd @ np.swapaxes(kd, -1, -2)
    a = np.maximum(s, 0.0) * np.tril(np.ones((T, T)))
    np.testing.assert_allclose(out, a @ vd, rtol=1e-12, atol=1e-13)


def _all_positive_inputs(T, D, seed):
    """q_i = c e0 + eps_i, k_j = c e0 + eps'_j with c^2 far above every tau, so
    every causal score exceeds its threshold and the ReLU never clips."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(1, 1, T, D, generator=g) * 0.1
    k = torch.randn(1, 1, T, D, generator=g) * 0.1
    q[..., 0] += 3.0
    k[..., 0] += 3.0
    v = torch.randn(1, 1, T, D, generator=g)
    return q, k, v


def _tau(i, beta, D):
    return beta * math.sqrt(2.0 * math.log(i + 1.0) / D)


def test_tra_all_positive_p1_prefix_sums():
    """No clipping, p = 1: out_i = q_i (sum_{j<=i} k_j v_j^T) - tau_i sum_{j<=i} v_j,
    evaluated with running prefix sums (an O(T D^2) algorithm, not the pair loop)."""
    T, D, beta = 50, 6, 1.3
    q, k, v = _all_positive_inputs(T, D, 20)
    out = oracle.tra_ref(q, k, v, beta, 1.0)[0, 0]
    qd, kd, vd = _f64(q)[0, 0], _f64(k)[0, 0], _f64(v)[0, 0]
    assert np.min((qd @ kd.T)[np.tril_indices(T)]) > _tau(T - 1, beta, D) + 1.0   # no clipping
    KV = np.zeros((D, D)); Vs = np.zeros(D)
    for i in range(T):
        KV += np.outer(kd[i], vd[i]); Vs += vd[i]
        np.testing.assert_allclose(out[i], qd[i] @ KV - _tau(i, beta, D) * Vs, rtol=1e-11, atol=1e-11)


def test_tra_all_positive_p2_prefix_sums():
    """No clipping, p = 2: (s - tau)^2 = s^2 - 2 tau s + tau^2 with s = q.k, so
    out_i = q_i^T (sum k k^T (x) v) q_i - 2 tau_i q_i (sum k v^T) + tau_i^2 sum v."""
    T, D, beta = 40, 5, 0.9
    q, k, v = _all_positive_inputs(T, D, 21)
    out = oracle.tra_ref(q, k, v, beta, 2.0)[0, 0]
    qd, kd, vd = _f64(q)[0, 0], _f64(k)[0, 0], _f64(v)[0, 0]
    KKV = np.zeros((D, D, D)); KV = np.zeros((D, D)); Vs = np.zeros(D)
    for i in range(T):
        KKV += np.einsum("a,b,c->abc", kd[i], kd[i], vd[i])
        KV += np.outer(kd[i], vd[i]); Vs += vd[i]
        t = _tau(i, beta, D)
        want = np.einsum("a,b,abc->c", qd[i], qd[i], KKV) - 2 * t * (qd[i] @ KV) + t * t * Vs
        np.testing.assert_allclose(out[i], want, rtol=1e-10, atol=1e-10)


def _tra_brute(q, k, v, beta, p):
    """Pure-Python loops over the definition (tiny inputs only)."""
    B, H, T, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    out = [[[[0.0] * D for _ in range(T)] for _ in range(H)] for _ in range(B)]
    for b, h, i in itertools.product(range(B), range(H), range(T)):
        tau = beta * math.sqrt(2.0 * math.log(i + 1) / D)
        for j in range(i + 1):
            x = sum(q[b][h][i][d] * k[b][h][j][d] for d in range(D)) - tau
            if x > 0:
                w = x ** p
                for d in range(D):
                    out[b][h][i][d] += w * v[b][h][j][d]
    return np.array(out)


@pytest.mark.parametrize("beta,p", [(0.0, 1.0), (0.7, 2.0), (0.4, 1.5), (-0.3, 3.0), (1.0, 0.5)])
def test_tra_bruteforce_tiny(beta, p):
    T, D = 11, 5
    q, k, v = _rand((1, 2, T, D), 30), _rand((1, 2, T, D), 31), _rand((1, 2, T, D), 32)
    want = _tra_brute(_f64(q).tolist(), _f64(k).tolist(), _f64(v).tolist(), beta, p)
    np.testing.assert_allclose(oracle.tra_ref(q, k, v, beta, p), want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("p", [1.0, 2.0, 1.5])
def test_tra_homogeneity_in_q(p):
    """beta = 0: scaling Q by c > 0 scales every score by c, the output by c^p."""
    q, k, v = inputs.tra_inputs(1, 2, 30, 16, dtype=torch.float32, seed=7)
    a = oracle.tra_ref(q, k, v, 0.0, p)
    b = oracle.tra_ref(q * 2.0, k, v, 0.0, p)
    np.testing.assert_allclose(b, (2.0 ** p) * a, rtol=1e-12, atol=1e-13)


def test_tra_linear_in_v():
    q, k, v1 = inputs.tra_inputs(1, 2, 30, 16, dtype=torch.float32, seed=8)
    v2 = _rand(v1.shape, 9)
    a = oracle.tra_ref(q, k, v1, 1.0, 2.0) + oracle.tra_ref(q, k, v2, 1.0, 2.0)
    np.testing.assert_allclose(oracle.tra_ref(q, k, v1 + v2, 1.0, 2.0), a, rtol=1e-6, atol=1e-6)


def test_tra_rows_subset_matches_full():
    q, k, v = inputs.tra_inputs(2, 2, 20, 8, dtype=torch.bfloat16, seed=4)
    full = oracle.tra_ref(q, k, v, 1.0, 2.0)
    rows = np.array([0, 19, 20, 39, 55, 79])
    sub = oracle.tra_ref(q, k, v, 1.0, 2.0, rows=rows)
    assert np.array_equal(sub, full.reshape(-1, 8)[rows])


def test_tra_bf16_inputs_widen_exactly():
    """bf16 inputs are read bit for bit: same values as the fp32 copy."""
    q, k, v = inputs.tra_inputs(1, 2, 16, 8, dtype=torch.bfloat16, seed=3)
    a = oracle.tra_ref(q, k, v, 1.0, 2.0)
    b = oracle.tra_ref(q.float(), k.float(), v.float(), 1.0, 2.0)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# NSA selection branch
# (openbox-llm page "nsa_selection_kernel.py": module docstring,
#  selection_forward_reference, lse in the query-outer kernel)
# --------------------------------------------------------------------------

def test_nsa_hand_example():
    with open(os.path.join(GOLDEN, "nsa_hand_T4_bs2.json")) as f:
        g = json.load(f)
    q, k, v = (_f32(g[n])[None, None] for n in ("q", "k", "v"))
    idx = np.asarray(g["block_idx"], dtype=np.int32)[None, None]
    out, lse = oracle.nsa_ref(q, k, v, idx, g["block_size"])
    np.testing.assert_allclose(out[0, 0], np.asarray(g["expected_out"]), rtol=1e-15, atol=0)
    np.testing.assert_allclose(lse[0, 0], np.asarray(g["expected_lse"]), rtol=1e-15, atol=0)
    assert out[0, 0, 3, 0] == 0.0 and lse[0, 0, 3] == -1e9


def _all_causal_blocks(B, Hkv, T, bs, S=None):
    nblk = T // bs
    S = nblk if S is None else S
    idx = np.full((B, Hkv, T, S), -1, dtype=np.int32)
    for i in range(T):
        c = i // bs
        idx[:, :, i, :c + 1] = np.arange(c + 1)
    return idx


def _dense_causal_reference(q, k, v, G):
    """torch fp64 scaled-dot-product attention with a causal mask (GQA by
    repeating each kv head G times) and the log-sum-exp of the scaled scores."""
    qd, kd, vd = q.double(), k.double().repeat_interleave(G, 1), v.double().repeat_interleave(G, 1)
    o = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, is_causal=True)
    T, D = q.shape[2], q.shape[3]
    s = (qd @ kd.transpose(-1, -2).contiguous()) / math.sqrt(D)
    s = s.masked_fill(~torch.ones(T, T, dtype=torch.bool).tril(), float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 1), (6, 2)])
def test_nsa_all_blocks_equals_dense_causal(Hq, Hkv):
    """Selecting every causally valid block gives dense causal softmax attention
    (G = 1), or dense GQA attention (G > 1)."""
    B, T, D, bs = 2, 256, 32, 16
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, dtype=torch.float32, seed=1)
    idx = _all_causal_blocks(B, Hkv, T, bs)
    out, lse = oracle.nsa_ref(q, k, v, idx, bs)
    ref_o, ref_lse = _dense_causal_reference(q, k, v, Hq // Hkv)
    np.testing.assert_allclose(out, ref_o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_nsa_empty_rows_exact():
    """Rows whose slots are all padding, all in the future, or all past the last
    block give exactly 0 and lse = -1e9."""
    B, Hq, Hkv, T, D, bs, S = 1, 4, 2, 64, 16, 8, 3
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, dtype=torch.float32, seed=2)
    idx = np.full((B, Hkv, T, S), -1, dtype=np.int32)
    for i in range(T):
        c = i // bs
        if i % 3 == 1:
            idx[0, :, i, :] = [c + 1, c + 2, -7] if c + 2 < T // bs else [-1, -2, -3]
        elif i % 3 == 2:
            idx[0, :, i, :] = [T // bs, T // bs + 5, 10 ** 6]
    out, lse = oracle.nsa_ref(q, k, v, idx, bs)
    assert np.all(out == 0.0)
    assert np.all(lse == -1e9)


def test_nsa_zero_q_counts_attended_tokens():
    """q = 0 makes the softmax uniform over A: lse = ln |A| (an integer count), and
    with v[j, d] = bit d of j, out[d] is the fraction of A with bit d set."""
    B, Hq, Hkv, T, D, bs, S = 1, 2, 1, 128, 8, 16, 4
    _, k, _ = inputs.nsa_inputs(B, Hq, Hkv, T, D, dtype=torch.float32, seed=3)
    q = torch.zeros(B, Hq, T, D)
    v = torch.tensor([[(j >> d) & 1 for d in range(D)] for j in range(T)], dtype=torch.float32)
    v = v[None, None]
    rng = np.random.default_rng(0)
    idx = rng.integers(-2, T // bs + 2, size=(B, Hkv, T, S)).astype(np.int32)
    out, lse = oracle.nsa_ref(q, k, v, idx, bs)
    for i in range(T):
        blocks = {int(b) for b in idx[0, 0, i] if 0 <= b < T // bs}
        A = sorted(j for b in blocks for j in range(b * bs, (b + 1) * bs) if j <= i)
        for h in range(Hq):
            if not A:
                assert lse[0, h, i] == -1e9 and np.all(out[0, h, i] == 0)
                continue
            assert round(math.exp(lse[0, h, i])) == len(A)
            assert abs(lse[0, h, i] - math.log(len(A))) < 1e-12
            frac = np.array([sum((j >> d) & 1 for j in A) / len(A) for d in range(D)])
            np.testing.assert_allclose(out[0, h, i], frac, rtol=1e-13, atol=1e-15)


def test_nsa_single_token():
    """Own block only and i at a block start: A = {i}, so out = v_i and
    lse = q_i . k_i / sqrt(D)."""
    B, Hq, Hkv, T, D, bs = 1, 4, 2, 64, 16, 8
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, dtype=torch.float32, seed=4)
    idx = np.full((B, Hkv, T, 2), -1, dtype=np.int32)
    idx[0, :, :, 0] = np.arange(T) // bs
    out, lse = oracle.nsa_ref(q, k, v, idx, bs)
    G = Hq // Hkv
    for i in range(0, T, bs):
        for h in range(Hq):
            kv = h // G
            assert np.array_equal(out[0, h, i], _f64(v)[0, kv, i])
            want = float(_f64(q)[0, h, i] @ _f64(k)[0, kv, i]) / math.sqrt(D)
            assert abs(lse[0, h, i] - want) < 1e-12


def test_nsa_group_heads_share_selection():
    """Copies of one query head inside a group give identical rows, and every
    head of a group reads the group's kv head (h // G)."""
    B, Hkv, G, T, D, bs, S = 1, 2, 3, 96, 16, 16, 4
    Hq = Hkv * G
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, dtype=torch.float32, seed=6)
    for kv in range(Hkv):
        q[:, kv * G + 1] = q[:, kv * G]
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=6)
    out, lse = oracle.nsa_ref(q, k, v, idx, bs)
    for kv in range(Hkv):
        assert np.array_equal(out[:, kv * G], out[:, kv * G + 1])
        assert np.array_equal(lse[:, kv * G], lse[:, kv * G + 1])
    # against a G = 1 problem built from one group's heads
    for h in range(Hq):
        kv = h // G
        o1, l1 = oracle.nsa_ref(q[:, h:h + 1], k[:, kv:kv + 1], v[:, kv:kv + 1],
                                idx[:, kv:kv + 1], bs)
        assert np.array_equal(out[:, h:h + 1], o1)
        assert np.array_equal(lse[:, h:h + 1], l1)


def test_nsa_slots_are_a_set():
    """Permuting the slots of a row, or repeating a slot, leaves the result as is."""
    B, Hq, Hkv, T, D, bs, S = 1, 2, 1, 128, 16, 16, 5
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, dtype=torch.float32, seed=7)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=7)
    out, lse = oracle.nsa_ref(q, k, v, idx, bs)
    rng = np.random.default_rng(1)
    perm = np.stack([rng.permutation(S) for _ in range(T)])
    idx_p = np.take_along_axis(idx, perm[None, None], axis=-1)
    out_p, lse_p = oracle.nsa_ref(q, k, v, idx_p, bs)
    assert np.array_equal(out, out_p) and np.array_equal(lse, lse_p)
    idx_d = np.concatenate([idx, idx[..., :2]], axis=-1)          # repeat two slots
    out_d, lse_d = oracle.nsa_ref(q, k, v, idx_d, bs)
    assert np.array_equal(out, out_d) and np.array_equal(lse, lse_d)


def test_nsa_lse_consistent_with_output():
    """sum_j exp(s_j - lse) = 1 and out = sum_j exp(s_j - lse) v_j over A."""
    B, Hq, Hkv, T, D, bs, S = 1, 2, 2, 64, 8, 8, 3
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, dtype=torch.float32, seed=8)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=8)
    out, lse = oracle.nsa_ref(q, k, v, idx, bs)
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    for h, i in itertools.product(range(Hq), range(T)):
        blocks = {int(b) for b in idx[0, h, i] if 0 <= b < T // bs}
        A = [j for b in sorted(blocks) for j in range(b * bs, (b + 1) * bs) if j <= i]
        w = np.exp(np.array([qd[0, h, i] @ kd[0, h, j] for j in A]) / math.sqrt(D) - lse[0, h, i])
        assert abs(w.sum() - 1.0) < 1e-12
        np.testing.assert_allclose(out[0, h, i], w @ vd[0, h, A], rtol=1e-11, atol=1e-12)


def _nsa_brute(q, k, v, idx, bs):
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nblk = T // bs
    out = np.zeros((B, Hq, T, D)); lse = np.full((B, Hq, T), -1e9)
    for b, h, i in itertools.product(range(B), range(Hq), range(T)):
        kv = h // G
        A = set()
        for blk in idx[b, kv, i]:
            if 0 <= blk < nblk:
                A |= {j for j in range(blk * bs, (blk + 1) * bs) if j <= i}
        if not A:
            continue
        s = {j: sum(float(q[b, h, i, d]) * float(k[b, kv, j, d]) for d in range(D)) / math.sqrt(D)
             for j in A}
        m = max(s.values())
        z = sum(math.exp(x - m) for x in s.values())
        for j in A:
            out[b, h, i] += math.exp(s[j] - m) / z * np.asarray(v[b, kv, j], dtype=np.float64)
        lse[b, h, i] = m + math.log(z)
    return out, lse


def test_nsa_bruteforce_tiny():
    B, Hq, Hkv, T, D, bs, S = 1, 4, 2, 16, 4, 4, 3
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, dtype=torch.bfloat16, seed=9)
    idx = np.random.default_rng(2).integers(-1, T // bs + 1, size=(B, Hkv, T, S)).astype(np.int32)
    out, lse = oracle.nsa_ref(q, k, v, idx, bs)
    wo, wl = _nsa_brute(_f64(q), _f64(k), _f64(v), idx, bs)
    np.testing.assert_allclose(out, wo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, wl, rtol=1e-13, atol=1e-13)


def test_nsa_rows_subset_matches_full():
    B, Hq, Hkv, T, D, bs, S = 1, 4, 2, 64, 16, 16, 3
    q, k, v = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=10)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=10)
    o, l = oracle.nsa_ref(q, k, v, idx, bs)
    rows = np.array([0, 63, 64, 130, 255])
    so, sl = oracle.nsa_ref(q, k, v, idx, bs, rows=rows)
    assert np.array_equal(so, o.reshape(-1, D)[rows]) and np.array_equal(sl, l.reshape(-1)[rows])


# --------------------------------------------------------------------------
# The seeded block_idx generator (input recipe, not method arithmetic)
# --------------------------------------------------------------------------

def test_block_idx_recipe():
    B, Hkv, T, bs, S = 1, 2, 2048, 64, 16
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=0)
    assert idx.dtype == np.int32 and idx.shape == (B, Hkv, T, S)
    for i in range(T):
        c = i // bs
        row = idx[0, 1, i]
        assert row[0] == c
        rest = row[1:]
        n = min(S - 1, c)
        assert np.all(rest[n:] == -1)
        picks = rest[:n]
        assert len(set(picks.tolist())) == n and np.all((picks >= 0) & (picks < c))
    assert np.array_equal(idx, inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=0))


def test_block_idx_recipe_more_slots_than_blocks():
    """S - 1 larger than the number of earlier blocks: every earlier block once."""
    idx = inputs.nsa_block_idx(1, 1, 320, 32, 16, seed=1)
    for i in range(320):
        c = i // 32
        row = idx[0, 0, i]
        assert row[0] == c
        assert sorted(row[1:1 + c].tolist()) == list(range(c))
        assert np.all(row[1 + c:] == -1)
