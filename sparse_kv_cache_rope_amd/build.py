"""Builds libfasa.so (HIP for gfx950) in-tree with hipcc.

    python sparse_kv_cache_rope_amd/build.py        # or build() from Python

Each source compiles to an object in parallel, then one link.  Always
rebuilds (the build is a few tens of seconds).
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfasa.so")
ROOT = os.path.dirname(HERE)

SOURCES = ["api.cpp", "rope_append.hip", "tip.hip", "topk.hip", "select2.hip", "attention.hip",
           "calibrate.hip", "probe.hip", "filter.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Wall", "-Wno-unused-result",
    # No packed-fp32 instructions in device code (the host pass warns that it
    # does not know the feature; that is harmless).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The hardware loads the first 16 dwords of kernel arguments into SGPRs
    # at wave launch, so a kernel's first loads need not wait for them.
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                sys.stderr.write(err)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
