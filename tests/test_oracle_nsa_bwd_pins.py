"""Pins for the NSA selection-branch backward oracle, checked on the CPU: torch
autograd of a plain fp64 dense formulation of the forward (masked softmax over the
selected causal tokens), autograd of torch's own scaled-dot-product attention when
every block is selected, central differences of the (separately pinned) forward
oracle, and the set semantics and empty-row behaviour the forward fixes."""
import numpy as np
import pytest
import torch

import oracle
from causal_attention_tiled_amd import inputs


def _dense_keep(idx, T, bs, G):
    """keep[b, h, i, j]: token j is attended by query i of head h -- the attended set
    of the page's forward (msb-msb/openbox-llm, "nsa_selection_kernel.py",
    `selection_forward_reference`: the tokens of the selected in-range blocks, each
    block once, causal j <= i, shared by the G heads of a kv group), built here as a
    Python set of token positions per (b, kv, i)."""
    B, Hkv = idx.shape[:2]
    keep = torch.zeros(B, Hkv * G, T, T, dtype=torch.bool)
    for b in range(B):
        for kv in range(Hkv):
            for i in range(T):
                tokens = set()
                for blk in np.asarray(idx[b, kv, i]).tolist():
                    if 0 <= blk < T // bs:
                        tokens.update(j for j in range(blk * bs, (blk + 1) * bs) if j <= i)
                if tokens:
                    keep[b, kv * G:(kv + 1) * G, i, sorted(tokens)] = True
    return keep


def _autograd(q, k, v, idx, bs, do):
    B, Hq, T, D = q.shape
    G = Hq // k.shape[1]
    Q, K, V = (x.double().clone().requires_grad_() for x in (q, k, v))
    Ke, Ve = K.repeat_interleave(G, dim=1), V.repeat_interleave(G, dim=1)
    s = (Q @ Ke.transpose(-1, -2)) * D ** -0.5
    keep = _dense_keep(idx, T, bs, G)
    s = s.masked_fill(~keep, float("-inf"))
    has = keep.any(-1, keepdim=True)
    p = torch.where(has, torch.softmax(torch.where(has, s, torch.zeros_like(s)), dim=-1),
                    torch.zeros_like(s))
    p = p * keep
    (p @ Ve).backward(do.double())
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


@pytest.mark.parametrize("G,bs,S", [(1, 4, 3), (4, 4, 2), (2, 8, 4)])
def test_nsa_bwd_matches_autograd(G, bs, S):
    B, Hkv, T, D = 1, 2, 32, 8
    q, k, v = inputs.nsa_inputs(B, Hkv * G, Hkv, T, D, dtype=torch.float32, seed=G + bs)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=bs)
    do = torch.randn(B, Hkv * G, T, D, generator=torch.Generator().manual_seed(3))
    got = oracle.nsa_bwd_ref(q, k, v, idx, bs, do)
    ref = _autograd(q, k, v, idx, bs, do)
    for g, r, n in zip(got, ref, ("dq", "dk", "dv")):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12, err_msg=n)


def test_nsa_bwd_all_blocks_is_causal_sdpa_gradient():
    """Every block selected: the gradient of torch's causal scaled-dot-product
    attention (GQA by repeating k, v), fp64."""
    B, G, Hkv, T, D, bs = 1, 2, 2, 24, 8, 4
    q, k, v = inputs.nsa_inputs(B, Hkv * G, Hkv, T, D, dtype=torch.float32, seed=7)
    nblk = T // bs
    idx = np.tile(np.arange(nblk, dtype=np.int32), (B, Hkv, T, 1))
    do = torch.randn(B, Hkv * G, T, D, generator=torch.Generator().manual_seed(8))
    got = oracle.nsa_bwd_ref(q, k, v, idx, bs, do)
    Q, K, V = (x.double().clone().requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        Q, K.repeat_interleave(G, 1), V.repeat_interleave(G, 1), is_causal=True)
    o.backward(do.double())
    for g, r, n in zip(got, (Q.grad, K.grad, V.grad), ("dq", "dk", "dv")):
        np.testing.assert_allclose(g, r.numpy(), rtol=1e-10, atol=1e-12, err_msg=n)


def test_nsa_bwd_central_differences_of_forward_oracle():
    B, G, Hkv, T, D, bs, S = 1, 2, 1, 16, 4, 4, 2
    q, k, v = inputs.nsa_inputs(B, Hkv * G, Hkv, T, D, dtype=torch.float32, seed=9)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=9)
    do = torch.randn(B, Hkv * G, T, D, generator=torch.Generator().manual_seed(10))
    dq, dk, dv = oracle.nsa_bwd_ref(q, k, v, idx, bs, do)
    h = 2.0 ** -12
    L = lambda qq, kk, vv: float(np.sum(oracle.nsa_ref(qq, kk, vv, idx, bs)[0] * do.double().numpy()))
    for which, grad, hd in ((0, dq, 1), (1, dk, 0), (2, dv, 0)):
        for (i, d) in ((0, 0), (5, 1), (11, 2), (15, 3)):
            t = [q.clone(), k.clone(), v.clone()]
            t[which][0, hd, i, d] += h
            up = L(*t)
            t[which][0, hd, i, d] -= 2 * h
            dn = L(*t)
            fd = (up - dn) / (2 * h)
            assert abs(fd - grad[0, hd, i, d]) <= 1e-6 * (1 + abs(fd)), (which, i, d, fd, grad[0, hd, i, d])


def test_nsa_bwd_set_semantics_and_empty_rows():
    """Repeating a slot changes nothing; a row whose slots are all padding gets dq = 0 and
    its dout reaches no dk, dv."""
    B, G, Hkv, T, D, bs, S = 1, 2, 1, 16, 8, 4, 3
    q, k, v = inputs.nsa_inputs(B, Hkv * G, Hkv, T, D, dtype=torch.float32, seed=11)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=11)
    do = torch.randn(B, Hkv * G, T, D, generator=torch.Generator().manual_seed(12))
    a = oracle.nsa_bwd_ref(q, k, v, idx, bs, do)
    dup = idx.copy()
    dup[..., 2] = dup[..., 0]
    dup2 = idx.copy()
    dup2[..., 2] = -1
    b = oracle.nsa_bwd_ref(q, k, v, dup, bs, do)
    c = oracle.nsa_bwd_ref(q, k, v, dup2, bs, do)
    for x, y in zip(b, c):
        assert np.array_equal(x, y)
    idx[0, 0, 9] = -1
    do2 = do.clone()
    do2[:, :, 9] *= 7.0
    e1 = oracle.nsa_bwd_ref(q, k, v, idx, bs, do)
    e2 = oracle.nsa_bwd_ref(q, k, v, idx, bs, do2)
    assert np.all(e1[0][:, :, 9] == 0.0)
    assert np.array_equal(e1[1], e2[1]) and np.array_equal(e1[2], e2[2])


def test_nsa_bwd_rows_subset_matches_full():
    B, G, Hkv, T, D, bs, S = 2, 2, 2, 16, 8, 4, 2
    q, k, v = inputs.nsa_inputs(B, Hkv * G, Hkv, T, D, dtype=torch.float32, seed=13)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=13)
    do = torch.randn(B, Hkv * G, T, D, generator=torch.Generator().manual_seed(14))
    full = oracle.nsa_bwd_ref(q, k, v, idx, bs, do)
    qr, kr = np.array([0, 17, 40, 63, 100, 127]), np.array([1, 15, 33, 47, 60])
    part = oracle.nsa_bwd_ref(q, k, v, idx, bs, do, qrows=qr, krows=kr)
    assert np.array_equal(part[0], full[0].reshape(-1, D)[qr])
    assert np.array_equal(part[1], full[1].reshape(-1, D)[kr])
    assert np.array_equal(part[2], full[2].reshape(-1, D)[kr])
