"""ctypes binding for ``libattn.so`` (C ABI in ``include/attn.h``).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and the current HIP stream are passed to the
C entry point of the same name, and a non-zero status becomes ``AttnError``.
There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libattn.so"
_lib = None


class AttnError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {attn_status_str(status)}")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load libattn.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.tra_fwd.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, cf, cf, vp]
    lib.tra_fwd.restype = ci
    lib.tra_fwd_f32.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, cf, cf, vp]
    lib.tra_fwd_f32.restype = ci
    lib.nsa_sel_bwd.argtypes = [vp] * 11 + [ctypes.c_size_t] + [ci] * 7 + [vp]
    lib.nsa_sel_fwd_fsa.argtypes = [vp] * 7 + [ctypes.c_size_t] + [ci] * 7 + [vp]
    lib.nsa_sel_fwd_fsa.restype = ci
    lib.nsa_sel_fsa_workspace_bytes.argtypes = [ci] * 7
    lib.nsa_sel_fsa_workspace_bytes.restype = ctypes.c_size_t
    lib.nsa_sel_bwd.restype = ci
    lib.nsa_sel_bwd_workspace_bytes.argtypes = [ci] * 7
    lib.nsa_sel_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.tra_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, cf, vp]
    lib.tra_bwd.restype = ci
    lib.tda_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                            ci, ci, ci, ci, cf, cf, cf, ci, vp]
    lib.tda_fwd.restype = ci
    lib.tda_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, cf, cf, ci, vp]
    lib.tda_fwd_noalloc.restype = ci
    lib.tda_noalloc_scratch_bytes.argtypes = []
    lib.tda_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.tda_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.tda_workspace_bytes.restype = ctypes.c_size_t
    lib.nsa_sel_fwd.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp]
    lib.nsa_sel_fwd.restype = ci
    lib.attn_status_str.argtypes = [ci]
    lib.attn_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def attn_status_str(status: int) -> str:
    return load_library().attn_status_str(int(status)).decode()


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _check(t: torch.Tensor, name: str, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _tra(fn_name: str, dtype, q, k, v, beta, p, out, stream):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dtype)
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must all be [B, H, T, D]")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", dtype)
    if out.shape != q.shape:
        raise ValueError("out must match q's shape")
    B, H, T, D = q.shape
    fn = getattr(load_library(), fn_name)
    rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            B, H, T, D, float(beta), float(p), _stream_handle(stream))
    if rc != 0:
        raise AttnError(fn_name, rc)
    return out


def tra_fwd(q, k, v, beta, p, out=None, stream=None):
    """Threshold Rectified Attention forward, bf16 in / bf16 out, fp32 accumulate.

    q, k, v: contiguous bfloat16 [B, H, T, D] on the GPU.  Returns ``out``.
    """
    return _tra("tra_fwd", torch.bfloat16, q, k, v, beta, p, out, stream)


def tra_fwd_f32(q, k, v, beta, p, out=None, stream=None):
    """Threshold Rectified Attention forward, fp32 in / fp32 out."""
    return _tra("tra_fwd_f32", torch.float32, q, k, v, beta, p, out, stream)


def tra_bwd(q, k, v, dout, beta, p, dq=None, dk=None, dv=None, stream=None):
    """Threshold Rectified Attention backward, bf16 in / bf16 out.

    q, k, v, dout: contiguous bfloat16 [B, H, T, D] on the GPU.  Returns (dq, dk, dv).
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _check(t, n, torch.bfloat16)
    if q.dim() != 4 or any(t.shape != q.shape for t in (k, v, dout)):
        raise ValueError("q, k, v, dout must all be [B, H, T, D]")
    grads = []
    for g, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if g is None:
            g = torch.empty_like(q)
        _check(g, n, torch.bfloat16)
        if g.shape != q.shape:
            raise ValueError(f"{n} must match q's shape")
        grads.append(g)
    B, H, T, D = q.shape
    rc = load_library().tra_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                *(g.data_ptr() for g in grads), B, H, T, D, float(beta),
                                float(p), _stream_handle(stream))
    if rc != 0:
        raise AttnError("tra_bwd", rc)
    return tuple(grads)


def tda_workspace_bytes(B, H, T, D, normalize=True) -> int:
    """Bytes of device workspace tda_fwd needs (0 without normalisation)."""
    return int(load_library().tda_workspace_bytes(B, H, T, D, 1 if normalize else 0))


def tda_fwd(q1, q2, k1, k2, v, beta, lam, p, normalize=True, out=None, workspace=None,
            stream=None):
    """Threshold Differential Attention forward, bf16 in / bf16 out.

    q1, q2, k1, k2, v: contiguous bfloat16 [B, H, T, D] on the GPU.  ``workspace``
    (uint8 GPU tensor of at least ``tda_workspace_bytes`` bytes) is allocated here
    when not given and normalisation needs it.  Returns ``out``.
    """
    for t, n in ((q1, "q1"), (q2, "q2"), (k1, "k1"), (k2, "k2"), (v, "v")):
        _check(t, n, torch.bfloat16)
    if q1.dim() != 4 or any(t.shape != q1.shape for t in (q2, k1, k2, v)):
        raise ValueError("q1, q2, k1, k2, v must all be [B, H, T, D]")
    if out is None:
        out = torch.empty_like(q1)
    _check(out, "out", torch.bfloat16)
    if out.shape != q1.shape:
        raise ValueError("out must match q1's shape")
    B, H, T, D = q1.shape
    need = tda_workspace_bytes(B, H, T, D, normalize)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q1.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _check(workspace, "workspace", workspace.dtype)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = load_library().tda_fwd(q1.data_ptr(), q2.data_ptr(), k1.data_ptr(), k2.data_ptr(),
                                v.data_ptr(), out.data_ptr(), ws_ptr, ws_bytes, B, H, T, D,
                                float(beta), float(lam), float(p), 1 if normalize else 0,
                                _stream_handle(stream))
    if rc != 0:
        raise AttnError("tda_fwd", rc)
    return out


def tda_noalloc_scratch_bytes() -> int:
    """Bytes of the static scratch that tda_fwd_noalloc uses (its size limit)."""
    return int(load_library().tda_noalloc_scratch_bytes())


def tda_fwd_noalloc(q1, q2, k1, k2, v, beta, lam, p, *, out, normalize=True, stream=None):
    """tda_fwd for callers that cannot allocate: the library keeps the normalised key
    rows in its own static scratch on the current GPU (calls that may overlap in time on
    one GPU race).  ``out`` (bfloat16, q1's shape) must be given.  Returns ``out``."""
    for t, n in ((q1, "q1"), (q2, "q2"), (k1, "k1"), (k2, "k2"), (v, "v"), (out, "out")):
        _check(t, n, torch.bfloat16)
    if q1.dim() != 4 or any(t.shape != q1.shape for t in (q2, k1, k2, v, out)):
        raise ValueError("q1, q2, k1, k2, v, out must all be [B, H, T, D]")
    B, H, T, D = q1.shape
    rc = load_library().tda_fwd_noalloc(q1.data_ptr(), q2.data_ptr(), k1.data_ptr(),
                                        k2.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, T, D,
                                        float(beta), float(lam), float(p),
                                        1 if normalize else 0, _stream_handle(stream))
    if rc != 0:
        raise AttnError("tda_fwd_noalloc", rc)
    return out


def nsa_sel_fwd(q, k, v, block_idx, block_size, out=None, lse=None, stream=None,
                want_lse: bool = True):
    """NSA selection-branch forward (bf16 in / out, fp32 lse).

    q: [B, Hq, T, D]; k, v: [B, Hkv, T, D]; block_idx: int32 [B, Hkv, T, S].
    Returns (out, lse) -- lse is None when ``want_lse`` is False and no buffer
    is given (the library then skips writing it).
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16)
    _check(block_idx, "block_idx", torch.int32)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, T, D]; k, v [B, Hkv, T, D]")
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != T or k.shape[3] != D:
        raise ValueError("k, v must be [B, Hkv, T, D] matching q")
    if block_idx.dim() != 4 or tuple(block_idx.shape[:3]) != (B, Hkv, T):
        raise ValueError("block_idx must be [B, Hkv, T, S]")
    S = block_idx.shape[3]
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", torch.bfloat16)
    if out.shape != q.shape:
        raise ValueError("out must match q's shape")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32)
        if tuple(lse.shape) != (B, Hq, T):
            raise ValueError("lse must be [B, Hq, T]")
    rc = load_library().nsa_sel_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    block_idx.data_ptr(), out.data_ptr(),
                                    lse.data_ptr() if lse is not None else None,
                                    B, Hq, Hkv, T, D, int(block_size), S,
                                    _stream_handle(stream))
    if rc != 0:
        raise AttnError("nsa_sel_fwd", rc)
    return out, lse


def nsa_sel_fsa_workspace_bytes(B, Hq, Hkv, T, D, block_size, S) -> int:
    """Bytes of device workspace nsa_sel_fwd_fsa needs."""
    return int(load_library().nsa_sel_fsa_workspace_bytes(B, Hq, Hkv, T, D, block_size, S))


def nsa_sel_fwd_fsa(q, k, v, block_idx, block_size, out=None, lse=None, workspace=None,
                    stream=None, want_lse: bool = True):
    """NSA selection-branch forward in block-outer form: the outputs of nsa_sel_fwd.

    Arguments as nsa_sel_fwd; ``workspace`` (uint8 GPU tensor of at least
    ``nsa_sel_fsa_workspace_bytes`` bytes) is allocated here when not given.
    Returns (out, lse).
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16)
    _check(block_idx, "block_idx", torch.int32)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, T, D]; k, v [B, Hkv, T, D]")
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != T or k.shape[3] != D:
        raise ValueError("k, v must be [B, Hkv, T, D] matching q")
    if block_idx.dim() != 4 or tuple(block_idx.shape[:3]) != (B, Hkv, T):
        raise ValueError("block_idx must be [B, Hkv, T, S]")
    S = block_idx.shape[3]
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", torch.bfloat16)
    if out.shape != q.shape:
        raise ValueError("out must match q's shape")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32)
        if tuple(lse.shape) != (B, Hq, T):
            raise ValueError("lse must be [B, Hq, T]")
    need = nsa_sel_fsa_workspace_bytes(B, Hq, Hkv, T, D, int(block_size), S)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(workspace, "workspace", torch.uint8)
    rc = load_library().nsa_sel_fwd_fsa(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        block_idx.data_ptr(), out.data_ptr(),
                                        lse.data_ptr() if lse is not None else None,
                                        workspace.data_ptr(), workspace.numel(),
                                        B, Hq, Hkv, T, D, int(block_size), S,
                                        _stream_handle(stream))
    if rc != 0:
        raise AttnError("nsa_sel_fwd_fsa", rc)
    return out, lse


def nsa_sel_bwd_workspace_bytes(B, Hq, Hkv, T, D, block_size, S) -> int:
    """Bytes of device workspace nsa_sel_bwd needs."""
    return int(load_library().nsa_sel_bwd_workspace_bytes(B, Hq, Hkv, T, D, block_size, S))


def nsa_sel_bwd(q, k, v, block_idx, block_size, out, lse, dout, dq=None, dk=None, dv=None,
                workspace=None, stream=None):
    """NSA selection-branch backward (bf16 in / out).

    q, out, dout: [B, Hq, T, D]; k, v: [B, Hkv, T, D]; block_idx: int32 [B, Hkv, T, S];
    lse: fp32 [B, Hq, T] (out and lse as returned by nsa_sel_fwd).  ``workspace`` (uint8
    GPU tensor of at least ``nsa_sel_bwd_workspace_bytes`` bytes) is allocated here when
    not given.  Returns (dq, dk, dv).
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _check(t, n, torch.bfloat16)
    _check(block_idx, "block_idx", torch.int32)
    _check(lse, "lse", torch.float32)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or out.shape != q.shape \
            or dout.shape != q.shape:
        raise ValueError("q, out, dout must be [B, Hq, T, D]; k, v [B, Hkv, T, D]")
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    if block_idx.dim() != 4 or tuple(block_idx.shape[:3]) != (B, Hkv, T):
        raise ValueError("block_idx must be [B, Hkv, T, S]")
    if tuple(lse.shape) != (B, Hq, T):
        raise ValueError("lse must be [B, Hq, T]")
    S = block_idx.shape[3]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for g, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _check(g, n, torch.bfloat16)
        if g.shape != ref.shape:
            raise ValueError(f"{n} has the wrong shape")
    if workspace is None:
        need = nsa_sel_bwd_workspace_bytes(B, Hq, Hkv, T, D, block_size, S)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(workspace, "workspace", workspace.dtype)
    rc = load_library().nsa_sel_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    block_idx.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), B, Hq, Hkv, T,
                                    D, int(block_size), S, _stream_handle(stream))
    if rc != 0:
        raise AttnError("nsa_sel_bwd", rc)
    return dq, dk, dv
