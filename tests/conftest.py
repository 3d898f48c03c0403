import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    if not gpu_available():
        pytest.skip("no GPU visible")
    import torch
    return torch.device("cuda:0")


@pytest.fixture(scope="session")
def nsa_c4_case():
    """NSA B=2 Hq=32 Hkv=4 T=4096 D=128 bs=64 S=16 (seed 0): inputs, block_idx and the
    oracle's output and lse on every row, computed once per session."""
    import oracle
    from causal_attention_tiled_amd import inputs
    c = inputs.CONFIGS["nsa_bf16_T4096_G8"]
    q, k, v = inputs.nsa_inputs(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], seed=0)
    idx = inputs.nsa_block_idx(c["B"], c["Hkv"], c["T"], c["block_size"], c["S"], seed=0)
    print("nsa T4096 G8: oracle on all 262144 rows", flush=True)
    ro, rl = oracle.nsa_ref(q, k, v, idx, c["block_size"])
    return dict(c=c, q=q, k=k, v=v, idx=idx, ref_o=ro, ref_lse=rl)


@pytest.fixture(scope="session")
def nsa_c5_case():
    """NSA B=1 Hq=64 Hkv=4 T=32768 D=128 bs=64 S=16 (seed 0): inputs, block_idx and the
    oracle's output and lse on all 2,097,152 rows (flat row ids in `rows`), computed once
    per session (about a minute of host time on 16 threads)."""
    import numpy as np
    import oracle
    from causal_attention_tiled_amd import inputs
    c = inputs.CONFIGS["nsa_bf16_T32768_G16"]
    q, k, v = inputs.nsa_inputs(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], seed=0)
    idx = inputs.nsa_block_idx(c["B"], c["Hkv"], c["T"], c["block_size"], c["S"], seed=0)
    B, Hq, T, D = q.shape
    rows = np.arange(B * Hq * T)
    print(f"nsa T32768 G16: oracle on all {rows.size} rows", flush=True)
    ro, rl = oracle.nsa_ref(q, k, v, idx, c["block_size"])
    return dict(c=c, q=q, k=k, v=v, idx=idx, rows=rows, ref_o=ro.reshape(-1, D),
                ref_lse=rl.reshape(-1))
