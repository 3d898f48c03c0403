"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerance for an output row (the D values of one (b, h, i)):
    |gpu - ref| <= rel * max_d |ref row| + rel * |ref|      elementwise,
with rel = 1e-2 for bf16 outputs and 1e-4 for fp32 outputs.  A reference row
that is all zero therefore demands an exact zero, unless the caller adds a floor
``floor * max |ref|`` (taken over the whole compared tensor) on the rows that
``floor_rows`` marks: rows whose exact result is zero only by cancellation of
terms the kernel rounds (the softmax gradient of a query that attends a single
key).  lse:
    |gpu - ref| <= 1e-3 * (1 + |ref|), and the empty-row sentinel -1e9 exactly.
"""
import numpy as np
import torch

BF16_REL = 1e-2
F32_REL = 1e-4
LSE_REL = 1e-3


def to_np(t):
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def assert_rows_close(gpu, ref, rel, what="", floor=0.0, floor_rows=None):
    """Elementwise row tolerance; with ``floor`` and ``floor_rows`` (a boolean mask over
    the leading dimensions, i.e. one flag per output row) the flagged rows get the extra
    absolute allowance floor * max|ref|."""
    g = to_np(gpu)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    bound = rel * np.abs(r).max(axis=-1, keepdims=True) + rel * np.abs(r)
    if floor and r.size:
        assert floor_rows is not None, "a floor needs the rows it applies to"
        fr = np.asarray(floor_rows, dtype=bool)
        assert fr.shape == r.shape[:-1], (fr.shape, r.shape)
        bound = bound + np.where(fr[..., None], floor * np.abs(r).max(), 0.0)
    err = np.abs(g - r)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} elements outside tolerance; first {idx[0].tolist()}, "
            f"worst {list(worst)}: gpu={g[worst]:.6g} ref={r[worst]:.6g} bound={bound[worst]:.3g}")


def assert_lse_close(gpu, ref, what=""):
    g = to_np(gpu)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape
    empty = r == -1e9
    assert np.all(g[empty] == np.float32(-1e9)), f"{what}: empty-row lse sentinel"
    ok = np.abs(g - r) <= LSE_REL * (1 + np.abs(r))
    ok |= empty
    if not ok.all():
        w = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {np.sum(~ok)} lse values off; first {w.tolist()}: "
                             f"gpu={g[tuple(w)]} ref={r[tuple(w)]}")


def sample_rows(B, H, T, n, seed=0, extra_positions=()):
    """Flat row ids (b*H + h)*T + i: every (b,h) gets the listed positions, plus n
    uniformly drawn rows overall."""
    rng = np.random.default_rng(seed)
    rows = []
    pos = [p for p in extra_positions if 0 <= p < T]
    for bh in range(B * H):
        rows.extend(bh * T + p for p in pos)
    rows.extend(rng.integers(0, B * H * T, size=n).tolist())
    return np.unique(np.asarray(rows, dtype=np.int64))
