"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of either method's arithmetic, so both the HIP path and the
oracle may be fed from it.

Workload shapes (no page measures on a dataset; these stand in for it):

* Threshold Rectified Attention: q, k ~ N(0, D^-1/2) elementwise (std D^-1/4),
  v ~ N(0, 1), drawn in the order q, k, v from one seeded CPU generator, then
  rounded to the storage dtype (bf16 round-to-nearest-even, or kept fp32).
* NSA selection: q, k, v ~ N(0, 1), same order and rounding.
* block_idx[b, kv, i, :] = the block that holds i (own block) first, then up
  to S-1 distinct blocks drawn uniformly without replacement from the blocks
  strictly before it, in draw order, then -1 padding.
"""
from __future__ import annotations

import numpy as np
import torch


def _draw(shape, std, gen):
    return torch.randn(*shape, generator=gen, dtype=torch.float32) * std


def tra_inputs(B: int, H: int, T: int, D: int, dtype=torch.bfloat16, seed: int = 0):
    """q, k, v [B, H, T, D] on the CPU, in ``dtype`` (bfloat16 or float32)."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    std_qk = float(D) ** -0.25
    q = _draw((B, H, T, D), std_qk, gen)
    k = _draw((B, H, T, D), std_qk, gen)
    v = _draw((B, H, T, D), 1.0, gen)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def tda_inputs(B: int, H: int, T: int, D: int, dtype=torch.bfloat16, seed: int = 0):
    """q1, q2, k1, k2, v [B, H, T, D] on the CPU: q and k rows N(0, D^-1/2) (so raw
    scores are about N(0, 1)), v N(0, 1); drawn in that order."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    std_qk = float(D) ** -0.25
    q1 = _draw((B, H, T, D), std_qk, gen)
    q2 = _draw((B, H, T, D), std_qk, gen)
    k1 = _draw((B, H, T, D), std_qk, gen)
    k2 = _draw((B, H, T, D), std_qk, gen)
    v = _draw((B, H, T, D), 1.0, gen)
    return tuple(t.to(dtype) for t in (q1, q2, k1, k2, v))


def nsa_inputs(B: int, Hq: int, Hkv: int, T: int, D: int, dtype=torch.bfloat16, seed: int = 0):
    """q [B, Hq, T, D], k, v [B, Hkv, T, D] on the CPU, N(0, 1), in ``dtype``."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    q = _draw((B, Hq, T, D), 1.0, gen)
    k = _draw((B, Hkv, T, D), 1.0, gen)
    v = _draw((B, Hkv, T, D), 1.0, gen)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def nsa_block_idx(B: int, Hkv: int, T: int, block_size: int, S: int, seed: int = 0,
                  chunk: int = 4096) -> np.ndarray:
    """int32 block_idx [B, Hkv, T, S]: own block, up to S-1 distinct earlier
    blocks drawn uniformly (random order), then -1 padding."""
    rng = np.random.default_rng(seed)
    nblk = max(T // block_size, 1)
    rows = B * Hkv * T
    out = np.full((rows, S), -1, dtype=np.int32)
    if S == 0 or rows == 0:
        return out.reshape(B, Hkv, T, S)
    pos = np.arange(rows, dtype=np.int64) % T
    own = pos // block_size
    out[:, 0] = own
    extra = S - 1
    if extra > 0:
        cols = np.arange(nblk)
        for r0 in range(0, rows, chunk):
            r1 = min(rows, r0 + chunk)
            c = own[r0:r1]                                   # candidates are 0 .. c-1
            keys = rng.random((r1 - r0, nblk))
            keys[cols[None, :] >= c[:, None]] = 2.0          # not a candidate
            width = min(extra, nblk)
            order = np.argsort(keys, axis=1, kind="stable")[:, :width]
            take = np.arange(width)[None, :] < np.minimum(c, width)[:, None]
            out[r0:r1, 1:1 + width] = np.where(take, order, -1).astype(np.int32)
    return out.reshape(B, Hkv, T, S)


# The workloads the library is measured and checked on.
CONFIGS = {
    "tra_f32_T256": dict(kind="tra", dtype="f32", B=1, H=2, T=256, D=64, beta=1.0, p=[2.0]),
    "tra_bf16_T2048_D64": dict(kind="tra", dtype="bf16", B=4, H=16, T=2048, D=64, beta=1.0,
                               p=[1.0, 2.0, 1.5]),
    "tra_bf16_T8192_D128": dict(kind="tra", dtype="bf16", B=2, H=32, T=8192, D=128, beta=1.0,
                                p=[2.0]),
    # Threshold Differential Attention at the T=8192 D=128 shape, normalised rows;
    # beta = D^-1/2 puts the thresholds at the same multiple of the cosines' spread
    # (D^-1/2) as beta = 1 does for the raw scores above.
    "tda_bf16_T8192_D128": dict(kind="tda", dtype="bf16", B=2, H=32, T=8192, D=128,
                                beta=128 ** -0.5, lam=0.5, p=[2.0], normalize=True),
    "nsa_bf16_T4096_G8": dict(kind="nsa", dtype="bf16", B=2, Hq=32, Hkv=4, T=4096, D=128,
                              block_size=64, S=16),
    "nsa_bf16_T32768_G16": dict(kind="nsa", dtype="bf16", B=1, Hq=64, Hkv=4, T=32768, D=128,
                                block_size=64, S=16),
}
