"""fp64 CPU oracle for the causal-attention forwards -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it, and it
shares no code with the HIP library: ``oracle.c`` is plain C compiled with gcc.

Functions
---------
``tra_ref(q, k, v, beta, p, rows=None)``
    Threshold Rectified Attention, out_i = sum_{j<=i} ReLU(q_i.k_j - tau_i)^p v_j,
    tau_i = beta*sqrt(2 ln(i+1)/D).  Source: snap-research/TDA page
    "triton_threshold_attention.py", module docstring and the forward kernel.
``tra_bwd_ref(q, k, v, dout, beta, p, qrows=None, krows=None)``
    Threshold Rectified Attention backward: (dq, dk, dv) in fp64 for the given
    query rows (dq) and key rows (dk, dv).  Source: the same page's backward
    kernels and autograd function (gradients of q, k, v).
``nsa_bwd_ref(q, k, v, block_idx, block_size, dout, qrows=None, krows=None)``
    NSA selection-branch backward: (dq, dk, dv) in fp64 for the given query rows
    (dq, flat (b*Hq + h)*T + i) and key rows (dk, dv, flat (b*Hkv + kv)*T + j).
    Built from the forward's definition (the page shows no backward).
``tda_ref(q1, q2, k1, k2, v, beta, lam, p, normalize=True, rows=None)``
    Threshold Differential Attention: optional L2 normalisation of the q and k
    rows, two Threshold Rectified Attention outputs over the same v, combined
    as out1 - clamp(lam, 0, 1) * out2.  Source: snap-research/TDA page
    "triton_threshold_attention.py", ``differential_threshold_rela_triton``.
``l2norm_ref(x)``
    The row normalisation of ``tda_ref``: x / max(||x||_2, 1e-12) with the norm rounded
    to the input dtype before the divide, as ``torch.nn.functional.normalize`` gives on
    a tensor of that dtype.
``nsa_ref(q, k, v, block_idx, block_size, rows=None)``
    NSA selection-branch forward (GQA softmax over the union of the selected
    blocks' causal tokens, scale D^-0.5), returning (out, lse).  Source:
    msb-msb/openbox-llm page "nsa_selection_kernel.py", module docstring,
    ``selection_forward_reference`` and the lse definition in the query-outer
    kernel.

Inputs are CPU ``torch`` tensors (float32 or bfloat16) or numpy arrays
(float32, or uint16 holding bf16 bits); they are read bit for bit and widened
exactly to float64 inside the C code.  ``rows`` optionally restricts the work
to a list of flat row ids ((b*H + h)*T + i); the result then has one row per
id, in that order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_F32, _BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.oracle_tra_rows.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64,
                                    dbl, dbl, vp, i64, vp, ctypes.c_int]
    lib.oracle_tra_rows.restype = ctypes.c_int
    lib.oracle_nsa_rows.argtypes = [vp, vp, vp, ctypes.c_int, vp, i64, i64, i64, i64, i64,
                                    i64, i64, vp, i64, vp, vp, ctypes.c_int]
    lib.oracle_nsa_rows.restype = ctypes.c_int
    lib.oracle_tda_rows.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64,
                                    dbl, dbl, dbl, ctypes.c_int, vp, i64, vp, ctypes.c_int]
    lib.oracle_tda_rows.restype = ctypes.c_int
    lib.oracle_tra_bwd_rows.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, dbl,
                                        dbl, vp, i64, vp, vp, i64, vp, vp, ctypes.c_int]
    lib.oracle_tra_bwd_rows.restype = ctypes.c_int
    lib.oracle_nsa_bwd_rows.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, i64, i64, i64, i64,
                                        i64, i64, i64, vp, i64, vp, vp, i64, vp, vp,
                                        ctypes.c_int]
    lib.oracle_nsa_bwd_rows.restype = ctypes.c_int
    lib.oracle_l2norm_rows.argtypes = [vp, ctypes.c_int, i64, i64, vp]
    lib.oracle_l2norm_rows.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    """OpenMP threads the oracle uses by default (OMP_NUM_THREADS or cores)."""
    return int(_load().oracle_num_threads())


def _as_input(x):
    """Return (contiguous numpy array, dtype code) holding x's exact bits."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), _BF16
            if x.dtype == torch.float32:
                return x.numpy(), _F32
            raise TypeError(f"oracle takes float32 or bfloat16, got {x.dtype}")
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, _F32
    if x.dtype == np.uint16:
        return x, _BF16
    raise TypeError(f"oracle takes float32 or bf16-bit uint16 arrays, got {x.dtype}")


def _rows_arg(rows):
    if rows is None:
        return None, None
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    return r, r.ctypes.data


def tra_ref(q, k, v, beta: float, p: float, rows=None, nthreads: int = 0) -> np.ndarray:
    """Threshold Rectified Attention forward in fp64.

    q, k, v: [B, H, T, D].  Returns float64 [B, H, T, D], or [len(rows), D].
    """
    qa, dt = _as_input(q)
    ka, dtk = _as_input(k)
    va, dtv = _as_input(v)
    if not (dt == dtk == dtv):
        raise TypeError("q, k, v must share one dtype")
    if not (qa.shape == ka.shape == va.shape) or qa.ndim != 4:
        raise ValueError("q, k, v must all be [B, H, T, D]")
    B, H, T, D = qa.shape
    r, rp = _rows_arg(rows)
    n = B * H * T if r is None else r.size
    out = np.zeros((n, D), dtype=np.float64)
    rc = _load().oracle_tra_rows(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, dt,
                                 B, H, T, D, float(beta), float(p), rp, n,
                                 out.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_tra_rows rejected its arguments")
    return out.reshape(B, H, T, D) if r is None else out


def tra_bwd_ref(q, k, v, dout, beta: float, p: float, qrows=None, krows=None,
                nthreads: int = 0):
    """Threshold Rectified Attention backward in fp64.

    q, k, v, dout: [B, H, T, D].  Returns (dq, dk, dv) as float64 [B, H, T, D] each, or,
    when qrows / krows are given, dq as [len(qrows), D] and dk, dv as [len(krows), D].
    """
    arrs = [_as_input(x) for x in (q, k, v, dout)]
    if len({a[1] for a in arrs}) != 1:
        raise TypeError("q, k, v, dout must share one dtype")
    if len({a[0].shape for a in arrs}) != 1 or arrs[0][0].ndim != 4:
        raise ValueError("q, k, v, dout must all be [B, H, T, D]")
    B, H, T, D = arrs[0][0].shape
    qr, qp = _rows_arg(qrows)
    kr, kp = _rows_arg(krows)
    nq = B * H * T if qr is None else qr.size
    nk = B * H * T if kr is None else kr.size
    dq = np.zeros((nq, D), dtype=np.float64)
    dk = np.zeros((nk, D), dtype=np.float64)
    dv = np.zeros((nk, D), dtype=np.float64)
    rc = _load().oracle_tra_bwd_rows(*(a[0].ctypes.data for a in arrs), arrs[0][1], B, H, T, D,
                                     float(beta), float(p), qp, nq, dq.ctypes.data, kp, nk,
                                     dk.ctypes.data, dv.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_tra_bwd_rows rejected its arguments")
    shape = (B, H, T, D)
    return (dq.reshape(shape) if qr is None else dq, dk.reshape(shape) if kr is None else dk,
            dv.reshape(shape) if kr is None else dv)


def nsa_bwd_ref(q, k, v, block_idx, block_size: int, dout, qrows=None, krows=None,
                nthreads: int = 0):
    """NSA selection-branch backward in fp64.

    q, dout: [B, Hq, T, D]; k, v: [B, Hkv, T, D]; block_idx: [B, Hkv, T, S] ints.
    Returns (dq, dk, dv): full float64 tensors, or per-row arrays when qrows / krows
    are given.
    """
    qa, dt = _as_input(q)
    ka, dtk = _as_input(k)
    va, dtv = _as_input(v)
    oa, dto = _as_input(dout)
    if not (dt == dtk == dtv == dto):
        raise TypeError("q, k, v, dout must share one dtype")
    if qa.ndim != 4 or ka.shape != va.shape or oa.shape != qa.shape:
        raise ValueError("q, dout must be [B, Hq, T, D]; k, v [B, Hkv, T, D]")
    B, Hq, T, D = qa.shape
    Hkv = ka.shape[1]
    idx = np.ascontiguousarray(np.asarray(block_idx, dtype=np.int32))
    if idx.ndim != 4 or idx.shape[:3] != (B, Hkv, T):
        raise ValueError("block_idx must be [B, Hkv, T, S]")
    S = idx.shape[3]
    qr, qp = _rows_arg(qrows)
    kr, kp = _rows_arg(krows)
    nq = B * Hq * T if qr is None else qr.size
    nk = B * Hkv * T if kr is None else kr.size
    dq = np.zeros((nq, D), dtype=np.float64)
    dk = np.zeros((nk, D), dtype=np.float64)
    dv = np.zeros((nk, D), dtype=np.float64)
    rc = _load().oracle_nsa_bwd_rows(qa.ctypes.data, ka.ctypes.data, va.ctypes.data,
                                     oa.ctypes.data, dt, idx.ctypes.data, B, Hq, Hkv, T, D,
                                     int(block_size), S, qp, nq, dq.ctypes.data, kp, nk,
                                     dk.ctypes.data, dv.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_nsa_bwd_rows rejected its arguments")
    if qr is None:
        dq = dq.reshape(B, Hq, T, D)
    if kr is None:
        dk, dv = dk.reshape(B, Hkv, T, D), dv.reshape(B, Hkv, T, D)
    return dq, dk, dv


def tda_ref(q1, q2, k1, k2, v, beta: float, lam: float, p: float, normalize: bool = True,
            rows=None, nthreads: int = 0) -> np.ndarray:
    """Threshold Differential Attention forward in fp64.

    q1, q2, k1, k2, v: [B, H, T, D].  Returns float64 [B, H, T, D], or [len(rows), D].
    """
    arrs = [_as_input(x) for x in (q1, q2, k1, k2, v)]
    dts = {a[1] for a in arrs}
    if len(dts) != 1:
        raise TypeError("q1, q2, k1, k2, v must share one dtype")
    shapes = {a[0].shape for a in arrs}
    if len(shapes) != 1 or arrs[0][0].ndim != 4:
        raise ValueError("q1, q2, k1, k2, v must all be [B, H, T, D]")
    B, H, T, D = arrs[0][0].shape
    r, rp = _rows_arg(rows)
    n = B * H * T if r is None else r.size
    out = np.zeros((n, D), dtype=np.float64)
    rc = _load().oracle_tda_rows(*(a[0].ctypes.data for a in arrs), dts.pop(),
                                 B, H, T, D, float(beta), float(lam), float(p),
                                 1 if normalize else 0, rp, n, out.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_tda_rows rejected its arguments")
    return out.reshape(B, H, T, D) if r is None else out


def l2norm_ref(x) -> np.ndarray:
    """The row normalisation that ``tda_ref(..., normalize=True)`` applies to q1, q2, k1
    and k2: each row over the last axis divided by its 2-norm rounded to the input dtype
    (at least 1e-12), each quotient rounded to the dtype.  Source: the page's
    ``differential_threshold_rela_triton`` normalises tensors of the input dtype with
    ``torch.nn.functional.normalize``.  Returns float64 of x's shape."""
    xa, dt = _as_input(x)
    D = xa.shape[-1]
    n = xa.size // D
    out = np.zeros((n, D), dtype=np.float64)
    if _load().oracle_l2norm_rows(xa.ctypes.data, dt, n, D, out.ctypes.data) != 0:
        raise ValueError("oracle_l2norm_rows rejected its arguments")
    return out.reshape(xa.shape)


def nsa_ref(q, k, v, block_idx, block_size: int, rows=None, nthreads: int = 0):
    """NSA selection-branch forward in fp64.

    q: [B, Hq, T, D]; k, v: [B, Hkv, T, D]; block_idx: [B, Hkv, T, S] ints.
    Returns (out, lse): float64 [B, Hq, T, D] and [B, Hq, T] (or per-row).
    """
    qa, dt = _as_input(q)
    ka, dtk = _as_input(k)
    va, dtv = _as_input(v)
    if not (dt == dtk == dtv):
        raise TypeError("q, k, v must share one dtype")
    try:
        import torch
        if isinstance(block_idx, torch.Tensor):
            block_idx = block_idx.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    idx = np.ascontiguousarray(np.asarray(block_idx).astype(np.int32))
    B, Hq, T, D = qa.shape
    Hkv = ka.shape[1]
    if ka.shape != (B, Hkv, T, D) or va.shape != ka.shape:
        raise ValueError("k, v must be [B, Hkv, T, D] matching q")
    if idx.ndim != 4 or idx.shape[:3] != (B, Hkv, T):
        raise ValueError("block_idx must be [B, Hkv, T, S]")
    S = idx.shape[3]
    r, rp = _rows_arg(rows)
    n = B * Hq * T if r is None else r.size
    out = np.zeros((n, D), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    rc = _load().oracle_nsa_rows(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, dt,
                                 idx.ctypes.data, B, Hq, Hkv, T, D, int(block_size), S,
                                 rp, n, out.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_nsa_rows rejected its arguments")
    if r is None:
        return out.reshape(B, Hq, T, D), lse.reshape(B, Hq, T)
    return out, lse
