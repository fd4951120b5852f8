"""Build libm2ssd.so (the gfx950 HIP library behind include/m2ssd.h) in-tree with hipcc.

    python selective_state_space_mixer_amd/build.py

(run it as a file: importing the package loads the library this script builds)
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libm2ssd.so")
SOURCES = ["api.cpp", "conv1d.hip", "ssd_scan.hip", "ssd_walk.hip", "ssd_step.hip", "gated_norm.hip", "stream_copy.hip", "ssd_bwd.hip"]
ARCH = os.environ.get("M2SSD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # keep the compiler from emitting packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if out.strip():
        sys.stderr.write(out + "\n")


def build(verbose: bool = True) -> str:
    """Compile every source for gfx950 and link libm2ssd.so (always rebuilds)."""
    with tempfile.TemporaryDirectory(prefix="m2ssd_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
            list(ex.map(_compile, SOURCES, objs))
        tmp_lib = LIB + ".tmp%d" % os.getpid()
        r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp_lib],
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout)
        os.replace(tmp_lib, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
