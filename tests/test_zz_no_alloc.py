"""tda_fwd_noalloc (the entry point for callers that cannot allocate: its scratch is a
static array inside the library) against tda_fwd with a caller workspace, through the
C ABI: two calls in a row on one GPU, the second with a smaller input, so the second
finds the first one's rows in the shared scratch."""
import pytest
import torch

import oracle
import causal_attention_tiled_amd as cat
from causal_attention_tiled_amd import inputs

from _parity import BF16_REL, assert_rows_close

pytestmark = pytest.mark.gpu


def test_tda_noalloc_matches_workspace_entry_point(gpu):
    for (B, H, T, D), p in (((2, 4, 1000, 128), 2.0), ((1, 2, 300, 64), 1.5)):
        print(f"tda_fwd_noalloc B{B} H{H} T{T} D{D} p={p}", flush=True)
        t5 = [x.to(gpu) for x in inputs.tda_inputs(B, H, T, D, seed=T + D)]
        ws = torch.empty(cat.tda_workspace_bytes(B, H, T, D), dtype=torch.uint8, device=gpu)
        a = cat.tda_fwd(*t5, 0.05, 0.5, p, workspace=ws)
        b = cat.tda_fwd_noalloc(*t5, 0.05, 0.5, p, out=torch.empty_like(t5[0]))
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        ref = oracle.tda_ref(*(x.cpu() for x in t5), 0.05, 0.5, p, normalize=True)
        assert_rows_close(b.cpu(), ref, BF16_REL, f"tda_fwd_noalloc T={T}")


def test_tda_noalloc_without_normalisation_uses_no_scratch(gpu):
    t5 = [x.to(gpu) for x in inputs.tda_inputs(1, 2, 200, 128, seed=7)]
    a = cat.tda_fwd(*t5, 0.5, 0.5, 2.0, normalize=False)
    b = cat.tda_fwd_noalloc(*t5, 0.5, 0.5, 2.0, normalize=False, out=torch.empty_like(t5[0]))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_tda_noalloc_refuses_more_than_its_scratch(gpu):
    z = torch.empty(1, 16, 8193, 128, dtype=torch.bfloat16, device=gpu)
    with pytest.raises(cat.AttnError) as e:
        cat.tda_fwd_noalloc(z, z, z, z, z, 0.05, 0.5, 2.0, out=torch.empty_like(z))
    assert e.value.status == -7
