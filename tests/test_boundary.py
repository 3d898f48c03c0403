"""The C ABI: libattn.so loads, exports every function include/attn.h declares,
and rejects bad arguments on the host before any HIP call (so these run on the
CPU: the dummy pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, ENULL, ESHAPE, EUNSUP, EALIGN, ELAUNCH, EWORK, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
P = 0x10000  # a 16-byte aligned dummy address (never touched by validation)


@pytest.fixture(scope="module")
def lib():
    import causal_attention_tiled_amd as cat
    if not os.path.exists(cat.library_path()):
        from causal_attention_tiled_amd import build
        build.build()
    return cat.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("tra_fwd", "tra_fwd_f32", "tra_bwd", "tda_fwd", "tda_workspace_bytes",
              "nsa_sel_fwd", "nsa_sel_bwd", "nsa_sel_bwd_workspace_bytes", "nsa_sel_fwd_fsa",
              "nsa_sel_fsa_workspace_bytes", "tda_fwd_noalloc", "tda_noalloc_scratch_bytes",
              "attn_status_str"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} is declared in attn.h but not exported"


def test_status_strings(lib):
    import causal_attention_tiled_amd as cat
    for code in (OK, ENULL, ESHAPE, EUNSUP, EALIGN, ELAUNCH, EWORK, ESCRATCH):
        assert cat.attn_status_str(code) not in ("", "unknown status")
    assert cat.attn_status_str(12345) == "unknown status"


def _tra(lib, fn, q=P, k=P, v=P, o=P, B=1, H=1, T=8, D=128, beta=1.0, p=2.0):
    return getattr(lib, fn)(q, k, v, o, B, H, T, D, beta, p, None)


@pytest.mark.parametrize("fn", ["tra_fwd", "tra_fwd_f32"])
def test_tra_validation(lib, fn):
    assert _tra(lib, fn, q=None) == ENULL
    assert _tra(lib, fn, o=None) == ENULL
    assert _tra(lib, fn, T=-1) == ESHAPE
    assert _tra(lib, fn, B=-2) == ESHAPE
    assert _tra(lib, fn, p=0.0) == ESHAPE
    assert _tra(lib, fn, p=-1.0) == ESHAPE
    assert _tra(lib, fn, p=float("nan")) == ESHAPE
    assert _tra(lib, fn, beta=float("inf")) == ESHAPE
    assert _tra(lib, fn, D=96) == EUNSUP
    assert _tra(lib, fn, D=256) == EUNSUP
    assert _tra(lib, fn, k=P + 8) == EALIGN
    assert _tra(lib, fn, o=P + 2) == EALIGN
    # empty problems are no-ops, even with NULL tensors
    assert _tra(lib, fn, q=None, k=None, v=None, o=None, B=0) == OK
    assert _tra(lib, fn, q=None, k=None, v=None, o=None, T=0) == OK
    # ...but the other arguments are still checked
    assert _tra(lib, fn, T=0, D=96) == EUNSUP


def _nsa(lib, q=P, k=P, v=P, idx=P, o=P, lse=P, B=1, Hq=8, Hkv=2, T=128, D=128, bs=64, S=4):
    return lib.nsa_sel_fwd(q, k, v, idx, o, lse, B, Hq, Hkv, T, D, bs, S, None)


def test_nsa_validation(lib):
    assert _nsa(lib, idx=None) == ENULL
    assert _nsa(lib, q=None) == ENULL
    assert _nsa(lib, Hq=6, Hkv=4) == ESHAPE          # Hq % Hkv
    assert _nsa(lib, Hkv=0) == ESHAPE
    assert _nsa(lib, T=100) == ESHAPE                # T % block_size
    assert _nsa(lib, S=0) == ESHAPE
    assert _nsa(lib, S=65) == EUNSUP
    assert _nsa(lib, bs=16) == EUNSUP
    assert _nsa(lib, bs=48) == EUNSUP
    assert _nsa(lib, D=32) == EUNSUP
    assert _nsa(lib, Hq=34, Hkv=2) == EUNSUP         # G = 17
    assert _nsa(lib, v=P + 4) == EALIGN
    assert _nsa(lib, idx=P + 2) == EALIGN
    assert _nsa(lib, lse=P + 1) == EALIGN
    assert _nsa(lib, q=None, k=None, v=None, idx=None, o=None, lse=None, T=0) == OK
    assert _nsa(lib, q=None, k=None, v=None, idx=None, o=None, lse=None, B=0) == OK


def _bwd(lib, q=P, k=P, v=P, do=P, dq=P, dk=P, dv=P, B=1, H=1, T=8, D=128, beta=1.0, p=2.0):
    return lib.tra_bwd(q, k, v, do, dq, dk, dv, B, H, T, D, beta, p, None)


def test_tra_bwd_validation(lib):
    assert _bwd(lib, do=None) == ENULL
    assert _bwd(lib, dq=None) == ENULL
    assert _bwd(lib, dv=None) == ENULL
    assert _bwd(lib, T=-1) == ESHAPE
    assert _bwd(lib, p=0.0) == ESHAPE
    assert _bwd(lib, beta=float("nan")) == ESHAPE
    assert _bwd(lib, D=32) == EUNSUP
    assert _bwd(lib, dk=P + 2) == EALIGN
    assert _bwd(lib, q=None, k=None, v=None, do=None, dq=None, dk=None, dv=None, B=0) == OK


def _tda(lib, q1=P, q2=P, k1=P, k2=P, v=P, o=P, ws=P, ws_bytes=1 << 40, B=1, H=1, T=8, D=128,
         beta=0.1, lam=0.5, p=2.0, norm=1):
    return lib.tda_fwd(q1, q2, k1, k2, v, o, ws, ws_bytes, B, H, T, D, beta, lam, p, norm, None)


def test_tda_validation(lib):
    assert lib.tda_workspace_bytes(2, 3, 5, 128, 1) == 2 * 2 * 3 * 5 * 128 * 2
    assert lib.tda_workspace_bytes(2, 3, 5, 128, 0) == 0
    assert lib.tda_workspace_bytes(-1, 3, 5, 128, 1) == 0
    assert _tda(lib, q2=None) == ENULL
    assert _tda(lib, k1=None) == ENULL
    assert _tda(lib, o=None) == ENULL
    assert _tda(lib, T=-1) == ESHAPE
    assert _tda(lib, lam=float("nan")) == ESHAPE
    assert _tda(lib, beta=float("inf")) == ESHAPE
    assert _tda(lib, p=-1.0) == ESHAPE
    assert _tda(lib, D=96) == EUNSUP
    assert _tda(lib, k2=P + 8) == EALIGN
    assert _tda(lib, ws=None) == EWORK
    assert _tda(lib, ws_bytes=2 * 8 * 128 * 2 - 1) == EWORK
    assert _tda(lib, ws=P + 4) == EALIGN
    # no normalisation needs no workspace; an empty problem is a no-op
    assert _tda(lib, q1=None, q2=None, k1=None, k2=None, v=None, o=None, ws=None, T=0) == OK


def _nbwd(lib, q=P, k=P, v=P, idx=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, ws=P, wsb=1 << 40,
          B=1, Hq=8, Hkv=2, T=128, D=128, bs=64, S=4):
    return lib.nsa_sel_bwd(q, k, v, idx, o, lse, do, dq, dk, dv, ws, wsb, B, Hq, Hkv, T, D, bs,
                           S, None)


def test_nsa_bwd_validation(lib):
    assert lib.nsa_sel_bwd_workspace_bytes(1, 8, 2, 128, 128, 64, 4) > 0
    assert lib.nsa_sel_bwd_workspace_bytes(1, 8, 2, 100, 128, 64, 4) == 0   # T % bs
    assert _nbwd(lib, o=None) == ENULL
    assert _nbwd(lib, lse=None) == ENULL
    assert _nbwd(lib, do=None) == ENULL
    assert _nbwd(lib, dk=None) == ENULL
    assert _nbwd(lib, idx=None) == ENULL
    assert _nbwd(lib, S=65) == EUNSUP
    assert _nbwd(lib, Hq=34, Hkv=2) == EUNSUP
    assert _nbwd(lib, T=100) == ESHAPE
    assert _nbwd(lib, ws=None) == EWORK
    assert _nbwd(lib, wsb=16) == EWORK
    assert _nbwd(lib, ws=P + 64) == EALIGN
    assert _nbwd(lib, dq=P + 8) == EALIGN
    assert _nbwd(lib, B=0, q=None, k=None, v=None, idx=None, o=None, lse=None, do=None,
                 dq=None, dk=None, dv=None, ws=None) == OK


def _fsa(lib, q=P, k=P, v=P, idx=P, o=P, lse=P, ws=P, wsb=1 << 40, B=1, Hq=8, Hkv=2, T=128,
         D=128, bs=64, S=4):
    return lib.nsa_sel_fwd_fsa(q, k, v, idx, o, lse, ws, wsb, B, Hq, Hkv, T, D, bs, S, None)


def test_nsa_fsa_validation(lib):
    small = lib.nsa_sel_fsa_workspace_bytes(1, 8, 2, 128, 128, 64, 4)
    assert small > 0
    assert lib.nsa_sel_fsa_workspace_bytes(1, 8, 2, 1024, 128, 64, 4) > small
    assert lib.nsa_sel_fsa_workspace_bytes(1, 8, 2, 100, 128, 64, 4) == 0   # T % bs
    assert _fsa(lib, o=None) == ENULL
    assert _fsa(lib, idx=None) == ENULL
    assert _fsa(lib, D=96) == EUNSUP
    assert _fsa(lib, bs=48, T=96) == EUNSUP
    assert _fsa(lib, S=65) == EUNSUP
    assert _fsa(lib, Hq=34, Hkv=2) == EUNSUP
    assert _fsa(lib, T=100) == ESHAPE
    assert _fsa(lib, ws=None) == EWORK
    assert _fsa(lib, wsb=small - 1) == EWORK
    assert _fsa(lib, ws=P + 64) == EALIGN
    assert _fsa(lib, o=P + 8) == EALIGN
    assert _fsa(lib, lse=P + 2) == EALIGN
    assert _fsa(lib, Hq=64, Hkv=4, T=131072) == EUNSUP   # q rows past 32-bit offsets
    # more (group, query, block) entries than int32 list positions hold
    assert _fsa(lib, B=1024, Hq=16, Hkv=16, T=8192, D=64, bs=32, S=64) == EUNSUP
    assert _nbwd(lib, B=1024, Hq=16, Hkv=16, T=8192, D=64, bs=32, S=64) == EUNSUP
    assert _fsa(lib, B=0, q=None, k=None, v=None, idx=None, o=None, lse=None, ws=None) == OK


def test_binding_refuses_cpu_tensors(lib):
    import torch
    import causal_attention_tiled_amd as cat
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        cat.tra_fwd(x, x, x, 1.0, 2.0)


def test_product_path_has_no_oracle_or_cpu_fallback():
    """Nothing in the package imports the oracle or computes on the CPU."""
    pkg = os.path.join(ROOT, "causal_attention_tiled_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            src = open(os.path.join(pkg, name)).read()
            assert not re.search(r"^\s*(import|from)\s+oracle\b", src, flags=re.M), name
            assert "liboracle" not in src, name


@pytest.mark.parametrize("D,T", [(128, 1 << 23), (64, 1 << 24), (128, (1 << 23) + 64)])
def test_bf16_slab_byte_limit(lib, D, T):
    """The bf16 kernels address one (batch, head) slab of T x D elements with 32-bit
    byte offsets: T * D * 2 >= 2^31 is refused before any HIP call."""
    assert _tra(lib, "tra_fwd", T=T, D=D) == EUNSUP
    assert _bwd(lib, T=T, D=D) == EUNSUP
    assert _tda(lib, T=T, D=D) == EUNSUP
    assert _nsa(lib, T=T, D=D, Hq=2, Hkv=2) == EUNSUP
    assert _nbwd(lib, T=T, D=D, Hq=2, Hkv=2) == EUNSUP
    assert _fsa(lib, T=T, D=D, Hq=2, Hkv=2) == EUNSUP


def _tdan(lib, q1=P, q2=P, k1=P, k2=P, v=P, o=P, B=1, H=1, T=8, D=128, beta=0.1, lam=0.5, p=2.0,
          norm=1):
    return lib.tda_fwd_noalloc(q1, q2, k1, k2, v, o, B, H, T, D, beta, lam, p, norm, None)


def test_tda_noalloc_validation(lib):
    """tda_fwd_noalloc: tda_fwd's checks, and a problem whose normalised keys exceed the
    static scratch is refused before any HIP call."""
    cap = lib.tda_noalloc_scratch_bytes()
    assert cap == 64 << 20
    assert _tdan(lib, q2=None) == ENULL
    assert _tdan(lib, o=None) == ENULL
    assert _tdan(lib, T=-1) == ESHAPE
    assert _tdan(lib, lam=float("nan")) == ESHAPE
    assert _tdan(lib, p=0.0) == ESHAPE
    assert _tdan(lib, D=96) == EUNSUP
    assert _tdan(lib, k1=P + 8) == EALIGN
    assert _tdan(lib, T=1 << 23) == EUNSUP
    # 2 * B*H*T*D * 2 bytes of normalised keys: 2^24 elements fit exactly, one row more does not
    assert lib.tda_workspace_bytes(1, 16, 8192, 128, 1) == cap
    assert _tdan(lib, B=1, H=16, T=8193, D=128) == ESCRATCH
    assert _tdan(lib, B=2, H=32, T=8192, D=128) == ESCRATCH
    assert _tdan(lib, q1=None, q2=None, k1=None, k2=None, v=None, o=None, T=0) == OK
