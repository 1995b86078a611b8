"""Builds libw8a8.so (gfx950) in-tree with hipcc.

Every HIP source is compiled with the flags below and linked into
``moe_token_amax_amd/libw8a8.so``. Objects go to ``moe_token_amax_amd/_build/``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libw8a8.so")
SOURCES = ["api.hip", "quant.hip", "prepack.hip", "gemm.hip", "mx.hip", "static.hip", "moe_io.hip", "w4a16.hip"]
ARCH = os.environ.get("W8A8_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # one IEEE rounding per fp32 operation: no fused multiply-add, subnormals kept
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def _hipcc() -> str:
    for p in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in p or os.path.exists(p):
            return p
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
