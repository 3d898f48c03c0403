"""Checks on the gfx950 assembly of the TRA backward's wide dk/dv kernel, compiled here
with hipcc and the library's flags (no GPU).  Its dK and dV products are MFMAs written as
inline assembly on accumulation-register tuples, so the compiler does not see their
hazards: no v_accvgpr_* instruction (a copy or read of those tuples, which would need
wait states after an MFMA writes them) may sit in a basic block that issues MFMAs, each
inline accumulation is preceded by its two wait states, and the accumulators are read
only after the long wait that follows the loop."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "causal_attention_tiled_amd")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def wide_kernels(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    sys.path.insert(0, PKG)
    try:
        import build as b
    finally:
        sys.path.pop(0)
    src = os.path.join(PKG, "csrc", "tra_bwd.hip")
    out = str(tmp_path_factory.mktemp("asm") / "tra_bwd.s")
    flags = [*b.CXXFLAGS, *b.EXTRA.get("tra_bwd.hip", [])]
    subprocess.run([hipcc, *flags, "--offload-device-only", "-S", src, "-o", out], check=True,
                   capture_output=True, timeout=600)
    text = open(out).read()
    kernels = {}
    for m in re.finditer(r"^(_Z\S*tra_bwd_dkv_wide_kernel\S*):", text, re.M):
        end = text.index(".Lfunc_end", m.end())
        kernels[m.group(1)] = text[m.end():end]
    return kernels


def _blocks(body):
    """Basic blocks as lists of instructions (comments and directives left out)."""
    blocks, cur = [], []
    for line in body.split("\n"):
        t = line.strip()
        if re.match(r"^\.LBB\S+:", t):
            blocks.append(cur)
            cur = []
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        cur.append(t)
    blocks.append(cur)
    return blocks


def test_one_kernel_per_power_mode(wide_kernels):
    assert len(wide_kernels) == 4, sorted(wide_kernels)


def test_no_accumulation_register_copies_next_to_the_mfmas(wide_kernels):
    for name, body in wide_kernels.items():
        for blk in _blocks(body):
            if any(i.startswith("v_mfma") for i in blk):
                acc = [i for i in blk if i.startswith("v_accvgpr")]
                assert not acc, (name, acc[:3])


def test_each_inline_accumulation_waits_two_states(wide_kernels):
    for name, body in wide_kernels.items():
        n = 0
        for blk in _blocks(body):
            for k, ins in enumerate(blk):
                if ins.startswith("v_mfma") and ins.split()[1].startswith("a["):
                    n += 1
                    assert k > 0 and blk[k - 1] == "s_nop 1", (name, blk[k - 1:k + 1])
        assert n > 0, name


def test_accumulators_read_only_after_the_final_wait(wide_kernels):
    """The wait after the loop (a run of s_nop worth at least 18 wait states) is there, and
    the blocks that read the accumulators out issue no MFMA.  (The reads sit in blocks
    after the wait; the text order of blocks is not their execution order, so this checks
    what the layout can show.)"""
    for name, body in wide_kernels.items():
        blocks = _blocks(body)
        best = 0
        for blk in blocks:
            run = 0
            for i in blk:
                m = re.match(r"s_nop (\d+)$", i)
                run = run + int(m.group(1)) + 1 if m else 0
                best = max(best, run)
        assert best >= 18, (name, best)
        readers = [blk for blk in blocks if any(i.startswith("v_accvgpr_read") for i in blk)]
        assert readers, name
        for blk in readers:
            assert not any(i.startswith("v_mfma") for i in blk), name
