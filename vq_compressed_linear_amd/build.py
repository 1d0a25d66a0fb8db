"""Builds libhxq.so for gfx950 in-tree with hipcc.

Usage: python -m vq_compressed_linear_amd.build  (or build() from Python).
The library lands next to this file; the Python binding loads it from there.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

try:
    from ._digest import source_digest
except ImportError:  # run as a script
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from vq_compressed_linear_amd._digest import source_digest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libhxq.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

SOURCES = ["hxq_gemv.hip", "hxq_gemv_mfma.hip", "hxq_gemv_mfma4.hip", "hxq_dequant.hip", "hxq_decode.hip", "hxq_decode1.hip", "hxq_gemm.hip", "hxq_gemm5.hip", "hxq_bwd.hip", "hxq_bwd_mfma.hip", "hxq_bwd_g5.hip", "hxq_api.cpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 vector instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, digest: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "--offload-arch=" + ARCH, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src == "hxq_api.cpp":
        cmd.insert(1, '-DHXQ_SOURCE_DIGEST="%s"' % digest)
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), res.stdout, res.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    digest = source_digest()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, digest), SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), res.stdout, res.stderr))
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
