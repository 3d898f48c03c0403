"""Benchmark of the fused causal-attention forwards on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

One step is one pass over both forwards of the hot path, each on its own
seeded synthetic batch already resident in HBM:
  * tra_fwd      Threshold Rectified Attention, bf16, B=2 H=32 T=8192 D=128,
                 beta=1, p=2 (useful FLOPs = 4*D per causal pair j <= i);
  * nsa_sel_fwd  NSA selection branch, bf16, B=1 Hq=64 Hkv=4 T=32768 D=128,
                 block_size=64, S=16 (gathered bytes = 2*block_size*D*2 per
                 valid selected block per (b, kv head, query)).
W untimed steps, then K timed steps between two device synchronisations.
Per-launch kernel durations come from HIP events recorded on the stream the
kernels run on.  After the timed steps, the other configurations of the method
(TRA at T=2048 D=64 for p = 1, 2, 1.5, 1.25; TRA fp32 at T=256; Threshold Differential
Attention at T=8192 D=128; the TRA backward at T=8192 D=128; NSA G=8 at T=4096;
NSA G=16 at T=32768 with caches flushed before each launch, the NSA backward and
block-outer forward at both NSA shapes) are timed on their own and reported under
"other_configs"; the rows beyond the two forwards (TDA, the TRA backward, the NSA
backward and block-outer forward) carry a "roofline" entry and, unless
--no-cpu-baseline, the oracle timed on a bounded sample as "cpu_baseline".  Prints ONE
JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import causal_attention_tiled_amd as cat  # noqa: E402
from causal_attention_tiled_amd import inputs  # noqa: E402

METRIC = ("useful causal-attn fwd TFLOP/s + % bf16 MFMA peak (T=8K,D=128); NSA fwd GB/s")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published

TRA = dict(B=2, H=32, T=8192, D=128, beta=1.0, p=2.0)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
CSRC = os.path.join(ROOT, "causal_attention_tiled_amd", "csrc")
# sources whose change invalidates a recorded traffic figure of each kernel
KERNEL_SOURCES = {
    "tra_fwd": ["tra_fwd.hip", "attn_internal.h", "attn_tile.h"],
    "nsa_sel_fwd": ["nsa_sel_fwd.hip", "attn_internal.h", "attn_tile.h"],
    "tda_fwd": ["tda_fwd.hip", "attn_internal.h", "attn_tile.h"],
    "tra_bwd": ["tra_bwd.hip", "attn_internal.h", "attn_tile.h"],
    "nsa_sel_bwd": ["nsa_sel_bwd.hip", "nsa_index.hip", "attn_internal.h", "attn_tile.h"],
    "nsa_sel_fwd_fsa": ["nsa_sel_fsa.hip", "nsa_index.hip", "attn_internal.h", "attn_tile.h"],
}
NSA = dict(B=1, Hq=64, Hkv=4, T=32768, D=128, block_size=64, S=16)


def tra_useful_flops(B, H, T, D, rows=None):
    """4*D flops (q.k and w*v) per causal pair; rows = flat ids, else all rows."""
    if rows is None:
        return 4.0 * D * B * H * T * (T + 1) / 2.0
    i = np.asarray(rows) % T
    return float(4.0 * D * np.sum(i + 1))


def nsa_gathered_bytes(idx, T, bs, D, rows_kv=None):
    """2 (K and V) * bs * D * 2 bytes per valid, distinct, causally reachable
    selected block per (b, kv head, query).  rows_kv: flat (b*Hkv+kv)*T+i ids."""
    nblk = T // bs
    flat = idx.reshape(-1, idx.shape[-1])
    if rows_kv is not None:
        flat = flat[np.asarray(rows_kv)]
        pos = np.asarray(rows_kv) % T
    else:
        pos = np.arange(flat.shape[0]) % T
    valid = (flat >= 0) & (flat < nblk) & (flat * bs <= pos[:, None])
    # distinct blocks only
    srt = np.sort(np.where(valid, flat, -1), axis=1)
    distinct = (srt >= 0) & np.concatenate([np.ones((srt.shape[0], 1), bool),
                                            srt[:, 1:] != srt[:, :-1]], axis=1)
    return float(distinct.sum()) * 2 * bs * D * 2


def nsa_tokens(idx, T, bs, rows_kv=None):
    """Attended tokens of each (b, kv head, query) row (flat (b*Hkv+kv)*T+i ids, else all
    rows): the j <= i of the row's distinct, in-range selected blocks."""
    nblk = T // bs
    flat = idx.reshape(-1, idx.shape[-1])
    if rows_kv is not None:
        flat = flat[np.asarray(rows_kv)]
        pos = (np.asarray(rows_kv) % T)[:, None]
    else:
        pos = (np.arange(flat.shape[0]) % T)[:, None]
    srt = np.sort(flat, axis=1)
    first = np.concatenate([np.ones((srt.shape[0], 1), bool), srt[:, 1:] != srt[:, :-1]], axis=1)
    ok = first & (srt >= 0) & (srt < nblk) & (srt * bs <= pos)
    return np.where(ok, np.minimum(bs, pos - srt * bs + 1), 0).sum(axis=1)


def nsa_useful_flops(idx, T, bs, D, G):
    """4*D FLOPs (q.k and p*v) per (query head, attended token)."""
    return 4.0 * D * G * float(nsa_tokens(idx, T, bs).sum())


def mfma_roofline(flops, ms, note):
    """Roofline entry of a kernel bound by the bf16 matrix units: useful FLOPs per launch
    over the launch time against the published dense peak."""
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": tf / PEAK_BF16_TFLOPS, "per_launch": note}


def oracle_rate(fn, budget_s, n0, nmax):
    """The fp64 oracle on growing samples: fn(n) draws n rows, runs the oracle on them and
    returns (seconds in the oracle call, work of those rows); n doubles until budget_s of
    oracle time is spent.  Returns (work per second, rows, seconds)."""
    n, spent, work, nrows = n0, 0.0, 0.0, 0
    while spent < budget_s and n <= nmax:
        s, w = fn(n)
        spent += s
        work += w
        nrows += n
        n *= 2
    return work / spent, nrows, spent


def oracle_entry(value, unit, sample):
    import oracle
    return {"value": value, "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
            "sample": sample}


def nsa_unique_bytes(B, Hq, Hkv, T, D, S):
    """Bytes every nsa_sel_fwd launch must move at least once: q, k, v, block_idx read,
    out and lse written."""
    return float(2 * B * Hkv * T * D * 2 + 2 * B * Hq * T * D * 2 + B * Hq * T * 4 + B * Hkv * T * S * 4)


def build_flags_text(path):
    """The compile-flag definitions of the build script (ARCH, CXXFLAGS, the per-file extra
    flags), # comments and blank lines left out: the part of it that decides the code a
    kernel compiles to."""
    import re
    with open(path) as fh:
        text = fh.read()
    parts = re.findall(r"^(?:ARCH = [^\n]*$|CXXFLAGS = \[.*?^\]|_THRESHOLD_FLAGS = \[.*?\]$"
                       r"|EXTRA = \{.*?\}$)", text, re.S | re.M)
    lines = (re.sub(r"#.*$", "", ln).rstrip() for p in parts for ln in p.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash(name):
    """Hash of the kernel's sources and of the build script's compile flags; in the C/HIP
    files, // comments and blank lines are left out, so an edit of a comment (or of how the
    build runs its compiles) keeps a measurement valid and any edit of code or flags
    invalidates it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            text = fh.read().decode()
        lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
        h.update("\n".join(ln for ln in lines if ln).encode())
    h.update(build_flags_text(os.path.join(CSRC, "..", "build.py")).encode())
    return h.hexdigest()[:16]


def recorded_traffic(name):
    """HBM bytes per launch recorded in profiles/hbm_traffic.txt for `name`, or None
    when there is no record or the kernel's sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    for line in open(TRAFFIC_FILE):
        if not line.startswith("kernel="):
            continue
        kv = dict(item.split("=", 1) for item in line.split())
        if kv.get("kernel") == name and kv.get("source") == kernel_source_hash(name):
            return float(kv["traffic_bytes"])
    return None


def cpu_baseline(q, k, v, idx_np, budget_s=12.0):
    """Time the fp64 oracle on bounded samples of both workloads."""
    import oracle
    threads = oracle.num_threads()
    rng = np.random.default_rng(123)
    B, H, T, D = TRA["B"], TRA["H"], TRA["T"], TRA["D"]
    # TRA: rows drawn uniformly, growing the sample until about budget_s/2 elapses
    n, spent, flops, nrows = 8, 0.0, 0.0, 0
    while spent < budget_s / 2 and n <= 1 << 16:
        rows = rng.integers(0, B * H * T, size=n)
        t0 = time.perf_counter()
        oracle.tra_ref(q, k, v, TRA["beta"], TRA["p"], rows=rows)
        spent += time.perf_counter() - t0
        flops += tra_useful_flops(B, H, T, D, rows)
        nrows += n
        n *= 2
    tra_tflops = flops / spent / 1e12
    return {"value": tra_tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{nrows} uniformly drawn rows of tra_fwd B=2 H=32 T=8192 D=128 p=2 "
                      f"({flops:.3g} useful FLOPs in {spent:.1f} s), fp64"}


def cpu_baseline_nsa(qn, kn, vn, idx_np, budget_s=8.0):
    import oracle
    rng = np.random.default_rng(321)
    B, Hq, Hkv, T, D, bs = NSA["B"], NSA["Hq"], NSA["Hkv"], NSA["T"], NSA["D"], NSA["block_size"]
    G = Hq // Hkv
    n, spent, nbytes, nrows = 64, 0.0, 0.0, 0
    while spent < budget_s and n <= 1 << 18:
        rows = rng.integers(0, B * Hq * T, size=n)
        t0 = time.perf_counter()
        oracle.nsa_ref(qn, kn, vn, idx_np, bs, rows=rows)
        spent += time.perf_counter() - t0
        bh = rows // T
        kv_rows = ((bh // Hq) * Hkv + (bh % Hq) // G) * T + rows % T
        nbytes += nsa_gathered_bytes(idx_np, T, bs, D, kv_rows) / G   # one head of G
        nrows += n
        n *= 2
    return {"value": nbytes / spent / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{nrows} uniformly drawn (head, query) rows of nsa_sel_fwd T=32768 G=16 "
                      f"({spent:.1f} s), fp64; bytes counted per head"}


def cpu_full(q, k, v, qn, kn, vn, idx_np):
    """The fp64 oracle over every row of both headline workloads, each in one timed call
    (wall clock): tra_fwd B2 H32 T8192 D128 p2 and nsa_sel_fwd B1 Hq64 Hkv4 T32768 G16."""
    import oracle
    out = {"cores": oracle.num_threads(), "kind": "oracle"}
    t0 = time.perf_counter()
    oracle.tra_ref(q, k, v, TRA["beta"], TRA["p"])
    s = time.perf_counter() - t0
    fl = tra_useful_flops(TRA["B"], TRA["H"], TRA["T"], TRA["D"])
    out["tra_fwd"] = {"s": s, "tflops": fl / s / 1e12, "rows": TRA["B"] * TRA["H"] * TRA["T"]}
    t0 = time.perf_counter()
    oracle.nsa_ref(qn, kn, vn, idx_np, NSA["block_size"])
    s = time.perf_counter() - t0
    gb = nsa_gathered_bytes(idx_np, NSA["T"], NSA["block_size"], NSA["D"])
    out["nsa_sel_fwd"] = {"s": s, "gathered_gbps": gb / s / 1e9,
                          "rows": NSA["B"] * NSA["Hq"] * NSA["T"]}
    return out


def time_launches(fn, warm, timed, between=None):
    """Per-launch durations (ms) of fn() from HIP events on the current stream;
    between() (not timed) runs before every launch when given."""
    for _ in range(warm):
        if between is not None:
            between()
        fn()
    torch.cuda.synchronize()
    ms = []
    for _ in range(timed):
        if between is not None:
            between()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    return ms


def stats(ms):
    return {"ms": float(np.mean(ms)), "ms_median": float(np.median(ms)), "ms_min": float(np.min(ms))}


def batch_ms(fn, n):
    """Mean duration of n back-to-back launches between two events (launch latency
    overlapped, as in a stream of work)."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / n


def timed(fn, warm=10, per_launch=20, batch=50):
    """Per-launch statistics, with "ms" the mean of a back-to-back batch."""
    st = stats(time_launches(fn, warm, per_launch))
    st["ms_per_launch_mean"] = st["ms"]
    st["ms"] = batch_ms(fn, batch)
    return st


def nsa_bwd_unique_bytes(B, Hq, Hkv, T, D, S):
    """Bytes every nsa_sel_bwd launch must move at least once: q, out, dout, lse, k, v and
    block_idx read, dq, dk, dv written."""
    return float(4 * B * Hq * T * D * 2 + 4 * B * Hkv * T * D * 2 + B * Hq * T * 4 + B * Hkv * T * S * 4)


def nsa_bwd(dev, q, k, v, gidx, bs, o, lse, gb, G, what, fwd_flops, warm=5, per_launch=10,
            batch=10):
    """Time nsa_sel_bwd on the forward's inputs; algorithmic bytes = the forward's gathered
    K/V bytes plus 2*G*D*2 bytes of q and dout per (group, query, block) visit.  Useful
    FLOPs: 10*D per (query head, attended token) (S, dP, dV, dK, dQ), i.e. 2.5x the
    forward's."""
    do = torch.randn(*q.shape, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).to(dev)
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    S = gidx.shape[-1]
    g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    ws = torch.empty(cat.nsa_sel_bwd_workspace_bytes(B, Hq, Hkv, T, D, bs, S), dtype=torch.uint8,
                     device=dev)
    st = timed(lambda: cat.nsa_sel_bwd(q, k, v, gidx, bs, o, lse, do, dq=g[0], dk=g[1], dv=g[2],
                                       workspace=ws), warm, per_launch, batch)
    total = gb * (1.0 + G / bs)
    fl = 2.5 * fwd_flops
    ub = nsa_bwd_unique_bytes(B, Hq, Hkv, T, D, S)
    roof = mfma_roofline(fl, st["ms"], f"{fl:.5g} useful FLOPs ({fl / PEAK_BF16_TFLOPS / 1e9:.4f} ms "
                         f"at peak) and {ub:.5g} unique bytes ({ub / PEAK_HBM_GBPS / 1e6:.4f} ms at peak)")
    return {what: dict(st, algorithmic_gb=total / 1e9, gbps=total / (st["ms"] * 1e-3) / 1e9,
                       workspace_gb=ws.numel() / 1e9, roofline=roof)}


def nsa_fsa(dev, q, k, v, gidx, bs, gb, what, flops, warm=5, per_launch=10, batch=20):
    """Time the block-outer forward (same outputs as nsa_sel_fwd) on the same inputs.  It
    reads each selected block once per list segment rather than once per query, so the
    query-outer kernel's gathered bytes are given for reference, not as its traffic."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    S = gidx.shape[-1]
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
    ws = torch.empty(cat.nsa_sel_fsa_workspace_bytes(B, Hq, Hkv, T, D, bs, S), dtype=torch.uint8,
                     device=dev)
    st = timed(lambda: cat.nsa_sel_fwd_fsa(q, k, v, gidx, bs, out=o, lse=lse, workspace=ws),
               warm, per_launch, batch)
    ub = nsa_unique_bytes(B, Hq, Hkv, T, D, S)
    roof = mfma_roofline(flops, st["ms"], f"{flops:.5g} useful FLOPs ({flops / PEAK_BF16_TFLOPS / 1e9:.4f} "
                         f"ms at peak) and {ub:.5g} unique bytes ({ub / PEAK_HBM_GBPS / 1e6:.4f} ms at peak)")
    return {what: dict(st, query_outer_gathered_gb=gb / 1e9, workspace_gb=ws.numel() / 1e9,
                       roofline=roof)}


def nsa_fwd_oracle_rate(cpu, fsa_entry, rng, budget_s=3.0):
    """The forward oracle (the function the block-outer form computes too) on bounded
    samples of the headline NSA workload (B1 Hq64 Hkv4 T32768 G16), in useful TFLOP/s at
    4*D per (query head, attended token)."""
    import oracle
    q, k, v, idx = cpu["q"], cpu["k"], cpu["v"], cpu["idx"]
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G, bs = Hq // Hkv, NSA["block_size"]

    def kv_rows(rows):
        bh = rows // T
        return ((bh // Hq) * Hkv + (bh % Hq) // G) * T + rows % T

    def fwd(n):
        rows = rng.integers(0, B * Hq * T, size=n)
        t0 = time.perf_counter()
        oracle.nsa_ref(q, k, v, idx, bs, rows=rows)
        return time.perf_counter() - t0, 4.0 * D * float(nsa_tokens(idx, T, bs, kv_rows(rows)).sum())
    rate, nrows, spent = oracle_rate(fwd, budget_s, 256, 1 << 18)
    fsa_entry["cpu_baseline"] = oracle_entry(
        rate / 1e12, "TFLOP/s", f"{nrows} uniformly drawn (head, query) rows of the same "
        f"workload through the forward oracle ({spent:.1f} s), fp64")


def tra_evaluated_weights(B, H, T, rows_per_wave=32, keys_per_tile=64):
    """Weights the forward kernel evaluates (epilogue elements): each wave of 32 query rows
    runs every 64-key tile up to the one holding its last row, masked keys included."""
    r0 = np.arange(0, T, rows_per_wave)
    last = np.minimum(r0 + rows_per_wave, T) - 1
    tiles = last // keys_per_tile + 1
    return float(B * H * rows_per_wave * keys_per_tile * tiles.sum())


def extra_configs(dev, nsa_c5=None, ceilings=None, cpu=None):
    """The other workloads of the method at their own sizes (not the headline line):
    TRA bf16 B4 H16 T2048 D64 at p = 1, 2, 1.5, 1.25; TRA fp32 B1 H2 T256 D64; TDA bf16
    B2 H32 T8192 D128 (normalised); the TRA backward at B2 H32 T8192 D128; NSA G=8
    at T=4096 (forward, block-outer forward and backward); both NSA forwards at B3
    Hq16 T8192 for G = 1, 2, 4, 8, 16; and NSA G=16 at T=32768:
    block-outer forward, backward, and forward with L2 and MALL flushed before every
    launch.  TDA, the TRA backward, the NSA backward and the block-outer NSA forward
    carry a roofline entry; with cpu (the headline NSA inputs on the host, or {} to skip
    the NSA rows) each also carries the oracle timed on a bounded sample of its rows, in
    the same unit."""
    if cpu is not None:
        import oracle  # the cpu_baseline entries only
    rng = np.random.default_rng(77)
    res = {}
    B, H, T, D = 4, 16, 2048, 64
    q, k, v = (x.to(dev) for x in inputs.tra_inputs(B, H, T, D, seed=0))
    out = torch.empty_like(q)
    fl = tra_useful_flops(B, H, T, D)
    for pw in (1.0, 2.0, 1.5, 1.25):
        st = timed(lambda: cat.tra_fwd(q, k, v, 1.0, pw, out=out), batch=200)
        tf = fl / (st["ms"] * 1e-3) / 1e12
        r = dict(st, tflops=tf, frac_bf16_peak=tf / PEAK_BF16_TFLOPS)
        if pw in (1.5, 1.25):
            # p = 1.5 costs one v_sqrt_f32 per evaluated weight, the general power one
            # v_log_f32 and one v_exp_f32 (transcendental-unit operations alike)
            ops = (1.0 if pw == 1.5 else 2.0) * tra_evaluated_weights(B, H, T)
            r["transcendental_ops"] = ops
            r["transcendental_ops_per_s"] = ops / (st["ms"] * 1e-3)
            if ceilings is not None:
                r["frac_of_measured_log_exp_rate"] = (r["transcendental_ops_per_s"] /
                                                      ceilings["log_exp_lane_ops_per_s"])
        res[f"tra_fwd B4 H16 T2048 D64 p{pw:g}"] = r
    q, k, v = (x.to(dev) for x in inputs.tra_inputs(1, 2, 256, 64, dtype=torch.float32, seed=0))
    out = torch.empty_like(q)
    res["tra_fwd_f32 B1 H2 T256 D64 p2"] = timed(
        lambda: cat.tra_fwd_f32(q, k, v, 1.0, 2.0, out=out), batch=200)
    c = inputs.CONFIGS["tda_bf16_T8192_D128"]
    B, H, T, D = c["B"], c["H"], c["T"], c["D"]
    t5c = inputs.tda_inputs(B, H, T, D, seed=0)
    t5 = [x.to(dev) for x in t5c]
    ws = torch.empty(cat.tda_workspace_bytes(B, H, T, D, c["normalize"]), dtype=torch.uint8,
                     device=dev)
    out = torch.empty_like(t5[0])
    fl = 6.0 * D * B * H * T * (T + 1) / 2.0      # two score products and one weighted sum per pair
    st = timed(lambda: cat.tda_fwd(*t5, c["beta"], c["lam"], 2.0, normalize=c["normalize"],
                                   out=out, workspace=ws), batch=20)
    tf = fl / (st["ms"] * 1e-3) / 1e12
    e = dict(st, tflops=tf, frac_bf16_peak=tf / PEAK_BF16_TFLOPS,
             roofline=mfma_roofline(fl, st["ms"], f"{fl:.5g} FLOPs (6*D per causal pair)"))
    if cpu is not None:
        def run(n):
            rows = rng.integers(0, B * H * T, size=n)
            t0 = time.perf_counter()
            oracle.tda_ref(*t5c, c["beta"], c["lam"], 2.0, normalize=c["normalize"], rows=rows)
            return time.perf_counter() - t0, 6.0 * D * float(np.sum(rows % T + 1))
        rate, nrows, spent = oracle_rate(run, 3.0, 64, 1 << 16)
        e["cpu_baseline"] = oracle_entry(
            rate / 1e12, "TFLOP/s", f"{nrows} uniformly drawn rows of the same workload "
            f"({spent:.1f} s, each call normalising every key row once), fp64")
    res["tda_fwd B2 H32 T8192 D128 normalised beta=D^-1/2 lambda=0.5 p2 (6D FLOP per pair)"] = e
    del t5, t5c, ws, out
    # TRA backward at the forward's measured shape
    B, H, T, D = 2, 32, 8192, 128
    qc, kc, vc = inputs.tra_inputs(B, H, T, D, seed=0)
    doc = torch.randn(B, H, T, D, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    q, k, v, do = (x.to(dev) for x in (qc, kc, vc, doc))
    g = [torch.empty_like(q) for _ in range(3)]
    fl = 10.0 * D * B * H * T * (T + 1) / 2.0     # five products per pair (S, dP, dV, dK, dQ)
    st = timed(lambda: cat.tra_bwd(q, k, v, do, 1.0, 2.0, dq=g[0], dk=g[1], dv=g[2]), 5, 10, 10)
    tf = fl / (st["ms"] * 1e-3) / 1e12
    e = dict(st, tflops=tf, frac_bf16_peak=tf / PEAK_BF16_TFLOPS,
             roofline=mfma_roofline(fl, st["ms"], f"{fl:.5g} FLOPs (10*D per causal pair)"))
    if cpu is not None:
        # n query rows (dq) and n key rows (dk, dv); a row's pairs count 5*D FLOPs on each
        # side, so that a full pass counts the 10*D per pair above
        def run(n):
            qr = rng.integers(0, B * H * T, size=n)
            kr = rng.integers(0, B * H * T, size=n)
            t0 = time.perf_counter()
            oracle.tra_bwd_ref(qc, kc, vc, doc, 1.0, 2.0, qrows=qr, krows=kr)
            pairs = float(np.sum(qr % T + 1) + np.sum(T - kr % T))
            return time.perf_counter() - t0, 5.0 * D * pairs
        rate, nrows, spent = oracle_rate(run, 3.0, 64, 1 << 15)
        e["cpu_baseline"] = oracle_entry(
            rate / 1e12, "TFLOP/s", f"{nrows} uniformly drawn query rows (dq) and as many key "
            f"rows (dk, dv) of the same workload ({spent:.1f} s), fp64")
    res["tra_bwd B2 H32 T8192 D128 beta1 p2 (10D FLOP per pair)"] = e
    del q, k, v, do, g, qc, kc, vc, doc
    B, Hq, Hkv, T, D, bs, S = 2, 32, 4, 4096, 128, 64, 16
    nsa_c4 = inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=0)
    qn, kn, vn = (x.to(dev) for x in nsa_c4)
    idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=0)
    gidx = torch.from_numpy(idx).to(dev)
    o = torch.empty_like(qn)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
    gb = nsa_gathered_bytes(idx, T, bs, D)
    fl = nsa_useful_flops(idx, T, bs, D, Hq // Hkv)
    st = timed(lambda: cat.nsa_sel_fwd(qn, kn, vn, gidx, bs, out=o, lse=lse), batch=50)
    res["nsa_sel_fwd B2 Hq32 Hkv4 T4096 D128 bs64 S16"] = dict(
        st, gathered_gb=gb / 1e9, gbps=gb / (st["ms"] * 1e-3) / 1e9,
        roofline=mfma_roofline(fl, st["ms"], f"{fl:.5g} useful FLOPs"))
    res.update(nsa_fsa(dev, qn, kn, vn, gidx, bs, gb,
                       "nsa_sel_fwd_fsa (block-outer) B2 Hq32 Hkv4 T4096 D128 bs64 S16", fl))
    kbwd = "nsa_sel_bwd B2 Hq32 Hkv4 T4096 D128 bs64 S16"
    res.update(nsa_bwd(dev, qn, kn, vn, gidx, bs, o, lse, gb, Hq // Hkv, kbwd, fl))
    if cpu is not None:
        # one call over every row: each call of the backward oracle first computes the
        # softmax statistics of every query row, which a sample of rows would not amortise
        doc = torch.randn(B, Hq, T, D, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
        t0 = time.perf_counter()
        oracle.nsa_bwd_ref(*nsa_c4, idx, bs, doc)
        spent = time.perf_counter() - t0
        res[kbwd]["cpu_baseline"] = oracle_entry(
            2.5 * fl / spent / 1e12, "TFLOP/s", f"the whole workload (every dq, dk and dv row) "
            f"in one call ({spent:.1f} s), fp64")
        del doc
    del qn, kn, vn, gidx, o, lse, nsa_c4
    # which NSA forward to call: both forms at B3 Hq16 T8192 D128 bs64 S16 over G = Hq/Hkv
    # (three batches, so that no launch shape coincides with the configurations above)
    B, Hq, T, D, bs, S = 3, 16, 8192, 128, 64, 16
    for Hkv in (16, 8, 4, 2, 1):
        qn, kn, vn = (x.to(dev) for x in inputs.nsa_inputs(B, Hq, Hkv, T, D, seed=0))
        idx = inputs.nsa_block_idx(B, Hkv, T, bs, S, seed=0)
        gidx = torch.from_numpy(idx).to(dev)
        o = torch.empty_like(qn)
        lse = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
        gb = nsa_gathered_bytes(idx, T, bs, D)
        st = timed(lambda: cat.nsa_sel_fwd(qn, kn, vn, gidx, bs, out=o, lse=lse), 5, 10, 20)
        shape = f"B3 Hq16 Hkv{Hkv} (G={Hq // Hkv}) T8192 D128 bs64 S16"
        res[f"nsa_sel_fwd {shape}"] = dict(st, gathered_gb=gb / 1e9,
                                           gbps=gb / (st["ms"] * 1e-3) / 1e9)
        fsa = nsa_fsa(dev, qn, kn, vn, gidx, bs, gb, f"nsa_sel_fwd_fsa (block-outer) {shape}",
                      nsa_useful_flops(idx, T, bs, D, Hq // Hkv))
        for v in fsa.values():
            v["query_outer_ms"] = st["ms"]
            v["speedup_over_query_outer"] = st["ms"] / v["ms"]
        res.update(fsa)
        del qn, kn, vn, gidx, o, lse
    if nsa_c5 is not None:
        fn, gb, t5, fl = nsa_c5
        kfsa = "nsa_sel_fwd_fsa (block-outer) B1 Hq64 Hkv4 T32768 D128 bs64 S16"
        kbwd = "nsa_sel_bwd B1 Hq64 Hkv4 T32768 D128 bs64 S16"
        res.update(nsa_fsa(dev, *t5[:5], gb, kfsa, fl, 3, 5, 5))
        res.update(nsa_bwd(dev, *t5, gb, NSA["Hq"] // NSA["Hkv"], kbwd, fl, 3, 5, 5))
        if cpu:
            nsa_fwd_oracle_rate(cpu, res[kfsa], rng)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        st = stats(time_launches(fn, 2, 8, between=lambda: flush.fill_(1)))
        res["nsa_sel_fwd B1 Hq64 Hkv4 T32768 D128 bs64 S16, cold (512 MiB written before each launch)"] = dict(
            st, gathered_gb=gb / 1e9, gbps=gb / (st["ms"] * 1e-3) / 1e9)
        del flush
    return res


def measured_ceilings():
    """Ceilings measured on this GPU by the probes in libprobes.so: streaming read
    bandwidth of a buffer served by L2 (16 MiB), by the memory-side cache (128 MiB) and
    by HBM (4 GiB); bf16 MFMA TFLOP/s with the engine clock seen during it; v_log_f32 +
    v_exp_f32 lane operations per second."""
    from causal_attention_tiled_amd import probes
    res = {}
    for name, nbytes in (("read_l2_gbps", 16 << 20), ("read_mall_gbps", 128 << 20),
                         ("read_hbm_gbps", 4 << 30)):
        res[name] = probes.read_bandwidth(nbytes)
    res["mfma_bf16_tflops"], res["sclk_ghz_under_mfma"] = probes.mfma_rate()
    res["log_exp_lane_ops_per_s"] = probes.transcendental_rate()
    res["note"] = ("read: 16-byte loads by 2048 workgroups of 256 threads, each XCD "
                   "re-reading its own contiguous eighth, of 16 MiB (L2-resident), 128 MiB "
                   "(MALL-resident) and 4 GiB (HBM); mfma: 4 chains of v_mfma_f32_32x32x16_bf16 per wave, 8 waves "
                   "per CU, clock = shader cycles (s_memtime) over 100 MHz ticks "
                   "(s_memrealtime); log/exp: 8 chains of v_log_f32, v_exp_f32 per lane")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="also time the oracle over every row of both headline workloads "
                         "(about a minute of host time)")
    ap.add_argument("--only", choices=["tra", "nsa"], default=None,
                    help="launch only one of the two forwards (for profiling runs)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="first run a plain device copy of this many bytes (3 times), the "
                         "reference for calibrating HBM traffic counters")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the timings of the other configurations")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the probe measurements of read, MFMA and log/exp ceilings")
    ap.add_argument("--source-hashes", action="store_true",
                    help="print the source hash of each kernel and exit")
    args = ap.parse_args()
    if args.source_hashes:
        for name in KERNEL_SOURCES:
            print(name, kernel_source_hash(name))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the forwards are single-GPU kernels; sharding is described, not run)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    cat.load_library()

    print("bench: generating inputs", file=sys.stderr, flush=True)
    q, k, v = inputs.tra_inputs(TRA["B"], TRA["H"], TRA["T"], TRA["D"], seed=0)
    qn, kn, vn = inputs.nsa_inputs(NSA["B"], NSA["Hq"], NSA["Hkv"], NSA["T"], NSA["D"], seed=0)
    idx_np = inputs.nsa_block_idx(NSA["B"], NSA["Hkv"], NSA["T"], NSA["block_size"], NSA["S"],
                                  seed=0)
    gq, gk, gv = q.to(dev), k.to(dev), v.to(dev)
    gqn, gkn, gvn = qn.to(dev), kn.to(dev), vn.to(dev)
    gidx = torch.from_numpy(idx_np).to(dev)
    out = torch.empty_like(gq)
    o_n = torch.empty_like(gqn)
    lse_n = torch.empty(NSA["B"], NSA["Hq"], NSA["T"], dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)          # reads and writes exactly copy_bytes
        torch.cuda.synchronize()
        del src, dst

    run_tra = args.only in (None, "tra")
    run_nsa = args.only in (None, "nsa")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if run_tra:
            cat.tra_fwd(gq, gk, gv, TRA["beta"], TRA["p"], out=out)
        if ev is not None:
            ev[1].record()
        if run_nsa:
            cat.nsa_sel_fwd(gqn, gkn, gvn, gidx, NSA["block_size"], out=o_n, lse=lse_n)
        if ev is not None:
            ev[2].record()

    print("bench: warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    tra_ms = [e[0].elapsed_time(e[1]) for e in events]
    nsa_ms = [e[1].elapsed_time(e[2]) for e in events]
    tra_avg = float(np.mean(tra_ms)) if run_tra else 0.0
    nsa_avg = float(np.mean(nsa_ms)) if run_nsa else 0.0

    flops = tra_useful_flops(TRA["B"], TRA["H"], TRA["T"], TRA["D"])
    gbytes = nsa_gathered_bytes(idx_np, NSA["T"], NSA["block_size"], NSA["D"])
    tra_tflops = flops / (tra_avg * 1e-3) / 1e12 if run_tra else 0.0
    nsa_gbps = gbytes / (nsa_avg * 1e-3) / 1e9 if run_nsa else 0.0

    roof_tra = {"kernel": "tra_fwd_bf16_kernel<128,p=2>", "bound": "mfma",
                "achieved": tra_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": tra_tflops / PEAK_BF16_TFLOPS, "traffic": recorded_traffic("tra_fwd"),
                "per_launch": f"{flops:.6g} useful FLOPs / {tra_avg:.4f} ms avg launch"}
    # NSA roofline: the larger of the time its useful FLOPs need at the bf16 MFMA peak and
    # the time its unique bytes need at the HBM peak (the gathered K/V is mostly served
    # from L2 and the memory-side cache, so gathered bytes over HBM bandwidth is no bound)
    G = NSA["Hq"] // NSA["Hkv"]
    nsa_flops = nsa_useful_flops(idx_np, NSA["T"], NSA["block_size"], NSA["D"], G)
    nsa_ubytes = nsa_unique_bytes(NSA["B"], NSA["Hq"], NSA["Hkv"], NSA["T"], NSA["D"], NSA["S"])
    t_flop_ms = nsa_flops / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    t_byte_ms = nsa_ubytes / (PEAK_HBM_GBPS * 1e9) * 1e3
    nsa_tflops = nsa_flops / (nsa_avg * 1e-3) / 1e12 if run_nsa else 0.0
    if t_flop_ms >= t_byte_ms:
        roof_nsa = {"kernel": "nsa_sel_fwd_kernel<128,64>", "bound": "mfma",
                    "achieved": nsa_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": nsa_tflops / PEAK_BF16_TFLOPS if run_nsa else 0.0}
    else:
        ubps = nsa_ubytes / (nsa_avg * 1e-3) / 1e9 if run_nsa else 0.0
        roof_nsa = {"kernel": "nsa_sel_fwd_kernel<128,64>", "bound": "hbm",
                    "achieved": ubps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": ubps / PEAK_HBM_GBPS}
    roof_nsa.update({
        "traffic": recorded_traffic("nsa_sel_fwd"),
        "per_launch": f"{nsa_flops:.6g} useful FLOPs ({t_flop_ms:.4f} ms at peak) and "
                      f"{nsa_ubytes:.6g} unique bytes ({t_byte_ms:.4f} ms at peak) / "
                      f"{nsa_avg:.4f} ms avg launch",
        "gathered_gbps": nsa_gbps,
        "gathered_note": f"{gbytes:.6g} gathered K/V bytes per launch (each selected block's "
                         "K and V once per GQA group) over the launch time; mostly served from "
                         "L2 and the memory-side cache, so not a fraction of HBM bandwidth"})
    dominant = roof_nsa if nsa_avg >= tra_avg else roof_tra
    ceilings = measured_ceilings() if not args.no_ceilings else None
    if ceilings is not None and run_nsa:
        # every gathered byte passes from L2 to the CUs: the measured L2 read rate bounds it
        roof_nsa["gathered_frac_of_l2_read_ceiling"] = nsa_gbps / ceilings["read_l2_gbps"]
        if roof_nsa.get("traffic"):
            rate = roof_nsa["traffic"] / (nsa_avg * 1e-3) / 1e9
            roof_nsa["l2_miss_gbps"] = rate
            roof_nsa["l2_miss_frac_of_mall_read_ceiling"] = rate / ceilings["read_mall_gbps"]

    result = {
        "metric": METRIC,
        "value": tra_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0, D^-1/2) q,k and N(0,1) v for tra_fwd; N(0,1) q,k,v and "
                "seeded random block lists (own block + 15 distinct earlier) for nsa_sel_fwd",
        "config": {"workload": "tra_fwd B2 H32 T8192 D128 beta1 p2 + nsa_sel_fwd B1 Hq64 Hkv4 "
                               "T32768 D128 bs64 S16",
                   "tra": TRA, "nsa": NSA},
        "tra_fwd": {"ms": tra_avg, "ms_median": float(np.median(tra_ms)),
                    "ms_min": float(np.min(tra_ms)), "tflops": tra_tflops,
                    "frac_bf16_peak": tra_tflops / PEAK_BF16_TFLOPS},
        "nsa_sel_fwd": {"ms": nsa_avg, "ms_median": float(np.median(nsa_ms)),
                        "ms_min": float(np.min(nsa_ms)), "gathered_gb": gbytes / 1e9,
                        "gathered_gbps": nsa_gbps,
                        "gathered_over_hbm_peak": nsa_gbps / PEAK_HBM_GBPS,
                        "useful_tflops": nsa_tflops,
                        "frac_bf16_peak": nsa_tflops / PEAK_BF16_TFLOPS,
                        "unique_gb": nsa_ubytes / 1e9},
        "roofline": dominant,
        "roofline_all": {"tra_fwd": roof_tra, "nsa_sel_fwd": roof_nsa},
    }
    if ceilings is not None:
        result["ceilings"] = ceilings
    if not args.no_extra and args.only is None:
        print("bench: other configurations", file=sys.stderr, flush=True)
        c5 = (lambda: cat.nsa_sel_fwd(gqn, gkn, gvn, gidx, NSA["block_size"], out=o_n, lse=lse_n),
              gbytes, (gqn, gkn, gvn, gidx, NSA["block_size"], o_n, lse_n), nsa_flops)
        cpu = None if args.no_cpu_baseline else dict(q=qn, k=kn, v=vn, idx=idx_np)
        result["other_configs"] = extra_configs(dev, nsa_c5=c5, ceilings=ceilings, cpu=cpu)
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(q, k, v, idx_np)
        result["cpu_baseline_nsa"] = cpu_baseline_nsa(qn, kn, vn, idx_np)
    if args.cpu_full:
        print("bench: oracle over the full workloads", file=sys.stderr, flush=True)
        result["cpu_full"] = cpu_full(q, k, v, qn, kn, vn, idx_np)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
