"""Build libspecverify.so (HIP, gfx950) in-tree with hipcc.

Each HIP source is compiled to an object in parallel, then linked into one
shared library next to this file.  Usage: ``python -m token_sampling_temp_amd.build``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "chain_reject.hip", "greedy_verify.hip", "softmax_renorm.hip", "gumbel_sample.hip",
           "fused_verify.hip", "d2t_expand.hip"]
# the benchmark's read-stream probe: a separate library, not part of the verification ABI
PROBE_SOURCE = "stream_probe.hip"
PROBE_PATH = os.path.join(HERE, "libsvprobe.so")

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link libspecverify.so (and the benchmark's libsvprobe.so);
    returns the library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + [PROBE_SOURCE]
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")), os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], LIB_PATH)
    _link(objs[-1:], PROBE_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build()
