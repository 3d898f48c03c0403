"""Host-side checks of bench.py (no GPU): the single-GPU refusal, the kernel source
hashes, and the reading of recorded HBM traffic (a figure is used only while the
kernel's code is the code it was measured on)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_source_hashes_cover_every_kernel():
    b = _bench()
    hashes = {n: b.kernel_source_hash(n) for n in b.KERNEL_SOURCES}
    assert set(hashes) >= {"tra_fwd", "nsa_sel_fwd", "tda_fwd", "tra_bwd", "nsa_sel_bwd",
                           "nsa_sel_fwd_fsa"}
    assert all(len(h) == 16 for h in hashes.values())


def test_recorded_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    b = _bench()
    h = b.kernel_source_hash("nsa_sel_fwd")
    f = tmp_path / "traffic.txt"
    f.write_text("# comment\n"
                 f"kernel=nsa_sel_fwd source={h} fetch_kib=1 write_kib=1 read_bytes=2 "
                 "write_bytes=3 traffic_bytes=5.5e+10\n"
                 "kernel=tra_fwd source=0000000000000000 traffic_bytes=1e9\n")
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(f))
    assert b.recorded_traffic("nsa_sel_fwd") == 5.5e10
    assert b.recorded_traffic("tra_fwd") is None          # measured on other code
    assert b.recorded_traffic("tda_fwd") is None          # never measured


def test_comment_edits_keep_the_hash(tmp_path, monkeypatch):
    """The hash ignores // comments and blank lines, and follows any code edit."""
    b = _bench()
    csrc = tmp_path / "csrc"             # the hash also reads csrc/../build.py
    csrc.mkdir()
    (csrc / "k.hip").write_text("int f() { return 1; }  // one\n\n")
    (tmp_path / "build.py").write_text("x = 1\n")
    monkeypatch.setattr(b, "CSRC", str(csrc))
    monkeypatch.setitem(b.KERNEL_SOURCES, "probe", ["k.hip"])
    h0 = b.kernel_source_hash("probe")
    (csrc / "k.hip").write_text("// a new comment\nint f() { return 1; }  // two\n")
    assert b.kernel_source_hash("probe") == h0
    (csrc / "k.hip").write_text("int f() { return 2; }\n")
    assert b.kernel_source_hash("probe") != h0


def test_build_flags_decide_the_hash(tmp_path, monkeypatch):
    """Of the build script, only the compile-flag definitions enter the hash: a change in
    how the build runs keeps it, a changed flag does not; the real script's flags are
    found."""
    b = _bench()
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    (csrc / "k.hip").write_text("int f() { return 1; }\n")
    script = ('ARCH = "gfx950"\nCXXFLAGS = [\n    "-O3",  # optimise\n    "-g0",\n]\n'
              '_THRESHOLD_FLAGS = ["-a", "-b"]\nEXTRA = {"k.hip": _THRESHOLD_FLAGS,\n'
              '         "m.hip": []}\n\n\ndef build():\n    return 1\n')
    monkeypatch.setattr(b, "CSRC", str(csrc))
    monkeypatch.setitem(b.KERNEL_SOURCES, "probe", ["k.hip"])
    (tmp_path / "build.py").write_text(script)
    h0 = b.kernel_source_hash("probe")
    (tmp_path / "build.py").write_text(script.replace("return 1", "return 2"))
    assert b.kernel_source_hash("probe") == h0
    for old, new in (('"-O3"', '"-O2"'), ('"-b"', '"-c"'), ('"m.hip": []', '"m.hip": ["-d"]'),
                     ('"gfx950"', '"gfx942"')):
        (tmp_path / "build.py").write_text(script.replace(old, new))
        assert b.kernel_source_hash("probe") != h0, old
    real = b.build_flags_text(os.path.join(ROOT, "causal_attention_tiled_amd", "build.py"))
    for piece in ("ARCH =", "CXXFLAGS =", "packed-fp32-ops", "_THRESHOLD_FLAGS =", "EXTRA =",
                  "tra_bwd.hip"):
        assert piece in real, piece


def test_nsa_token_counts():
    """The work counts of the NSA rows: the attended tokens of each query row match a direct
    count on a tiny case with duplicates, padding, ids past the end and a block after the
    query, for all rows and for a subset."""
    import numpy as np
    b = _bench()
    T, bs, G = 12, 4, 3
    idx = np.full((1, 2, T, 3), -1, dtype=np.int32)
    rng = np.random.default_rng(5)
    for kv in range(2):
        for i in range(T):
            idx[0, kv, i] = rng.integers(-1, T // bs + 1, size=3)
    idx[0, 0, 5] = [1, 1, 2]                  # duplicate, and block 2 starts after query 5
    direct = []
    for kv in range(2):
        for i in range(T):
            blocks = {int(x) for x in idx[0, kv, i] if 0 <= x < T // bs}
            direct.append(sum(1 for j in range(i + 1) if j // bs in blocks))
    tokens = b.nsa_tokens(idx, T, bs)
    assert tokens.tolist() == direct
    assert b.nsa_tokens(idx, T, bs, [5, 17]).tolist() == [direct[5], direct[17]]
    assert b.nsa_useful_flops(idx, T, bs, 64, G) == 4.0 * 64 * G * sum(direct)
