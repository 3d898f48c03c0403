"""Microbenchmarks of MI355X ceilings used by the rooflines in bench.py (libprobes.so,
built next to libattn.so by ``causal_attention_tiled_amd.build``; not part of the
attention library's C ABI).

``read_bandwidth(nbytes)``  streaming read GB/s of a buffer of nbytes, each XCD reading
                            its own contiguous eighth: 16 MiB (2 MiB per XCD) is served by
                            the XCDs' L2s, 128 MiB (16 MiB per XCD) by the memory-side
                            cache (MALL), 4 GiB by HBM.
``mfma_rate()``             bf16 MFMA TFLOP/s (v_mfma_f32_32x32x16_bf16 chains) and the
                            engine clock observed meanwhile (GHz).
``mfma_chain_rate(chains)``  bf16 MFMA TFLOP/s of one wave per SIMD running 1, 2 or 4
                            independent chains of dependent MFMAs.
``transcendental_rate()``   v_log_f32 + v_exp_f32 instructions per second (lane ops).
``lds_rate(mode)``          LDS read TB/s over the chip, and bytes per shader clock per
                            compute unit, of ds_read_b128 (mode 0) or ds_read_b64_tr_b16 (1).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprobes.so")
_lib = None
_CUS = 256  # compute units of an MI355X


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run python -m causal_attention_tiled_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.probe_read.argtypes = [vp, i64, ctypes.c_int, ctypes.c_int, vp, vp]
        lib.probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp]
        lib.probe_trans.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
        lib.probe_mfma_chains.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
        lib.probe_mfma_chains.restype = ctypes.c_int
        lib.probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        lib.probe_lds.restype = ctypes.c_int
        for f in (lib.probe_read, lib.probe_mfma, lib.probe_trans):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _time_ms(launch, reps):
    import torch
    launch()                                   # warm caches and clocks
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        launch()
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    return best


def read_bandwidth(nbytes: int, passes: int = 0, reps: int = 5) -> float:
    """Best-of-reps GB/s of `passes` streaming reads of an nbytes buffer (8 workgroups
    of 256 threads per compute unit)."""
    import torch
    lib = _load()
    if passes <= 0:
        passes = max(1, int(2e9 // nbytes))
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        rc = lib.probe_read(buf.data_ptr(), buf.numel() * 4, passes, 8 * _CUS, sink.data_ptr(),
                            stream)
        if rc != 0:
            raise RuntimeError(f"probe_read failed: {rc}")
    ms = _time_ms(launch, reps)
    return nbytes * passes / (ms * 1e-3) / 1e9


def mfma_rate(iters: int = 20000, reps: int = 3):
    """(TFLOP/s, GHz): 2 workgroups of 4 waves per compute unit, each wave 4 chains of
    32x32x16 bf16 MFMAs; the clock is the median over waves of shader cycles over
    100 MHz ticks."""
    import torch
    lib = _load()
    grid = 2 * _CUS
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2 * 4 * grid, dtype=torch.int64, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        rc = lib.probe_mfma(iters, grid, sink.data_ptr(), clk.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"probe_mfma failed: {rc}")
    ms = _time_ms(launch, reps)
    flops = 4.0 * 32768 * iters * 4 * grid
    c = clk.view(-1, 2).double()
    ghz = float((c[:, 0] / c[:, 1]).median()) * 0.1
    return flops / (ms * 1e-3) / 1e12, ghz


def mfma_chain_rate(chains: int, iters: int = 20000, reps: int = 3) -> float:
    """bf16 TFLOP/s of one wave per SIMD (1024 single-wave workgroups) running `chains`
    independent chains of dependent 32x32x16 MFMAs."""
    import torch
    lib = _load()
    grid = 4 * _CUS
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        rc = lib.probe_mfma_chains(iters, chains, grid, sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"probe_mfma_chains failed: {rc}")
    ms = _time_ms(launch, reps)
    return 32768.0 * iters * chains * grid / (ms * 1e-3) / 1e12


def transcendental_rate(iters: int = 4000, reps: int = 3) -> float:
    """v_log_f32 + v_exp_f32 lane operations per second (8 workgroups of 256 per CU)."""
    import torch
    lib = _load()
    grid = 8 * _CUS
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        rc = lib.probe_trans(iters, grid, sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"probe_trans failed: {rc}")
    ms = _time_ms(launch, reps)
    return 2.0 * 8 * iters * 256 * grid / (ms * 1e-3)


def lds_rate(mode: int, iters: int = 20000, reps: int = 3):
    """(TB/s over the chip, bytes per shader clock per compute unit) of LDS reads: 4
    workgroups of 4 waves per compute unit, 8 reads per wave per iteration (mode 0:
    ds_read_b128, 1 KiB per read; mode 1: ds_read_b64_tr_b16, 512 bytes).  The clock is
    the median over waves of shader cycles over 100 MHz ticks during the loop."""
    import torch
    lib = _load()
    grid = 4 * _CUS
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    clk = torch.zeros(2 * 4 * grid, dtype=torch.int64, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        rc = lib.probe_lds(iters, mode, grid, sink.data_ptr(), clk.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"probe_lds failed: {rc}")
    ms = _time_ms(launch, reps)
    per_read = 1024 if mode == 0 else 512
    total = float(per_read) * 8 * iters * 4 * grid
    c = clk.view(-1, 2).double()
    ghz = float((c[:, 0] / c[:, 1]).median()) * 0.1
    tbps = total / (ms * 1e-3) / 1e12
    return tbps, tbps * 1e12 / _CUS / (ghz * 1e9)
