"""Build libfa.so (the C-ABI attention library) in-tree with hipcc, for
gfx950 only, and libfacalib.so (the streaming-read kernel that calibrates
the HBM byte counters for profiling).  Usage:
python -m exact_tiled_attention_10_amd.build"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfa.so")
CALIB_OUT = os.path.join(HERE, "libfacalib.so")
CALIB_SOURCE = "fa_calib.hip"
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_pad.hip", "fa_fwd_fp8.hip", "fa_noalloc.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ALU forms stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Kernel sources only: they never form a NaN (masked scores are -inf and every
# -inf - -inf is guarded; probabilities recomputed from the saved LSE are
# clamped to [0, 1] by the exponential's output clamp, so a masked key's score
# cannot overflow into inf * 0), so the max reductions need no NaN
# canonicalisation.
# The C-ABI front end keeps full IEEE semantics (it rejects NaN scales).
KERNEL_FLAGS = ["-fno-honor-nans"]
# Per-source extras.  The decode kernel keeps its accumulators in VGPRs:
# with AGPR accumulators the compiler copies all of them between the two
# register files on every loop iteration.
SOURCE_FLAGS: dict = {"fa_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def compile_flags(src: str) -> list:
    """hipcc flags for one source file (without -c / -o)."""
    extra = KERNEL_FLAGS if src.endswith(".hip") else []
    return [*FLAGS, *extra, *SOURCE_FLAGS.get(src, [])]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *compile_flags(src), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs = list(ex.map(_compile, SOURCES + [CALIB_SOURCE]))
    _link(objs[:-1], OUT)
    _link(objs[-1:], CALIB_OUT)
    if verbose:
        print(f"built {OUT} and {CALIB_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
