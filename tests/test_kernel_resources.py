"""Compile-time resource checks of the gfx950 kernels (CPU only, no GPU).

A kernel whose register arrays get demoted to scratch memory runs several
times slower without any error, so every kernel's private segment is bounded
here: a few spilled registers outside a hot loop are tolerated, array-sized
scratch is not.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_token_amax_amd", "csrc")
MAX_SCRATCH = 64  # bytes per lane


def _hipcc():
    p = "/opt/rocm/bin/hipcc"
    return p if os.path.exists(p) else shutil.which("hipcc")


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src", ["quant.hip", "prepack.hip", "gemm.hip", "mx.hip"])
def test_kernels_use_no_array_scratch(src, tmp_path):
    from moe_token_amax_amd._build import FLAGS
    cmd = [_hipcc(), *FLAGS, "--cuda-device-only", "-c", os.path.join(CSRC, src), "-o",
           str(tmp_path / "k.o"), "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", r.stderr)
    scratch = [int(v) for v in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    assert names and len(names) == len(scratch)
    bad = {n: s for n, s in zip(names, scratch) if s > MAX_SCRATCH}
    assert not bad, f"kernels with array-sized scratch: {bad}"
