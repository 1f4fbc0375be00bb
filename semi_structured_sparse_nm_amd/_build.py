"""Build the HIP library libnmsparse.so (gfx950) in-tree with hipcc.

Every csrc/*.hip file is compiled to an object under _build/ (in parallel),
then linked into semi_structured_sparse_nm_amd/libnmsparse.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnmsparse.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed fp32 arithmetic stays off (device code only; the host pass warns)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off",
]


def _headers():
    return glob.glob(os.path.join(CSRC, "*.hpp")) + [os.path.join(ROOT, "include", "nm_sparse.h")]


def _compile(src: str, force: bool = True) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if not force and os.path.exists(obj):
        newest = max(os.path.getmtime(f) for f in [src, *_headers()])
        if os.path.getmtime(obj) > newest:
            return obj
    t0 = time.time()
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    print(f"  {os.path.basename(src)}: {time.time() - t0:.0f} s", flush=True)
    return obj


def build(jobs: int = 8, force: bool = True) -> str:
    """Compile the HIP sources (every one, or with force=False only those
    older than their object) and link libnmsparse.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda f: _compile(f, force), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--changed" not in sys.argv))
