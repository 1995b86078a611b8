"""Compile-time resource checks of the gfx950 kernels (CPU only, no GPU).

A kernel whose register arrays get demoted to scratch memory runs several
times slower without any error, so every kernel's private segment is bounded
here (a few spilled registers outside the hot loops are tolerated, array-sized
scratch is not), and the innermost loops that issue MFMAs may not touch
scratch memory at all.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_token_amax_amd", "csrc")
MAX_SCRATCH = 128  # bytes per lane
SOURCES = ["quant.hip", "prepack.hip", "gemm.hip", "mx.hip", "static.hip", "moe_io.hip", "w4a16.hip"]


def _hipcc():
    p = "/opt/rocm/bin/hipcc"
    return p if os.path.exists(p) else shutil.which("hipcc")


def _flags():
    # _build.py on its own (importing the package would load the library)
    import importlib.util
    spec = importlib.util.spec_from_file_location("w8a8_build", os.path.join(ROOT, "moe_token_amax_amd",
                                                                           "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return [*mod.FLAGS, "--cuda-device-only", "-I" + CSRC]


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_kernels_use_no_array_scratch(src, tmp_path):
    cmd = [_hipcc(), *_flags(), "-c", os.path.join(CSRC, src), "-o", str(tmp_path / "k.o"),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", r.stderr)
    scratch = [int(v) for v in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    assert names and len(names) == len(scratch)
    bad = {n: s for n, s in zip(names, scratch) if s > MAX_SCRATCH}
    assert not bad, f"kernels with array-sized scratch: {bad}"


def _innermost_mfma_loops(lines):
    """(start, end) line ranges of loops (a label and a later branch back to it)
    that contain an MFMA and no smaller such loop."""
    labels = {}
    for i, ln in enumerate(lines):
        m = re.match(r"^(\.LBB\d+_\d+):", ln)
        if m:
            labels[m.group(1)] = i
    loops = []
    for i, ln in enumerate(lines):
        m = re.search(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\d+_\d+)", ln)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            a = labels[m.group(1)]
            if any("v_mfma" in x for x in lines[a:i + 1]):
                loops.append((a, i))
    return [(a, b) for a, b in loops
            if not any((c, d) != (a, b) and a <= c and d <= b for c, d in loops)]


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src", ["gemm.hip", "mx.hip", "w4a16.hip"])
def test_mfma_loops_do_not_touch_scratch(src, tmp_path):
    out = tmp_path / "k.s"
    r = subprocess.run([_hipcc(), *_flags(), "-S", os.path.join(CSRC, src), "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    bad = []
    checked = 0
    functions = set(re.findall(r"^\s*\.type\s+(\S+),@function", asm, re.M))
    for m in re.finditer(r"^(_Z\S+):\s*(?:;.*)?$", asm, re.M):
        if m.group(1) not in functions:
            continue  # a data symbol (device array)
        body = asm[m.end():]
        body = body[:body.index(".Lfunc_end")]
        lines = body.split("\n")
        for a, b in _innermost_mfma_loops(lines):
            checked += 1
            n = sum(1 for x in lines[a:b + 1] if "scratch_" in x)
            if n:
                bad.append((m.group(1)[:60], n))
    assert checked > 0
    assert not bad, f"scratch accesses inside MFMA loops: {bad}"
