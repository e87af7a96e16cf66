"""Build libdsa.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m sparse_attention_scores_amd.build

Every source under csrc/ is compiled for gfx950 only and linked into
``sparse_attention_scores_amd/libdsa.so``.  Packed-FP32 instructions are
disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdsa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs: with them in AGPRs the compiler copies
    # the whole attention accumulator set through VALU moves every key tile
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str) -> str:
    cmd = [hipcc(), *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    return warn


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for src, warn in zip(srcs, ex.map(_compile, srcs, objs)):
            if warn.strip() and verbose:
                print(f"[{os.path.basename(src)}]\n{warn}", file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probe()
    return LIB


PROBE_SRC = os.path.join(HERE, "probe", "peaks.hip")
PROBE_LIB = os.path.join(HERE, "probe", "libdsa_probe.so")


def build_probe() -> str:
    """The measurement harness's calibration kernels (a streaming copy and
    an MFMA-only loop), in a library of their own beside libdsa."""
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *COMMON, "-shared", "-o", tmp, PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose=True))
