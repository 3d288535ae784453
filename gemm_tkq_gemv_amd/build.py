"""Builds libtkq.so (hand-written HIP for gfx950) in place, next to this file.

    python -m gemm_tkq_gemv_amd.build          # compile every source, link

Each ``csrc/*.hip`` is compiled with ``hipcc --offload-arch=gfx950 -O3`` (IEEE
division and square root, no fast-math; packed-fp32 instruction generation
disabled) into ``_build/`` and linked into ``gemm_tkq_gemv_amd/libtkq.so``.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtkq.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-I" + os.path.join(ROOT, "include"),
    # no packed fp32 (v_pk_*_f32) instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (p.stdout + p.stderr).splitlines()
            if "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln]
    if p.returncode:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(msgs)))
    return obj, msgs


def build(verbose=False):
    """Compile every HIP source for gfx950 and link libtkq.so.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for _, msgs in results:
        if verbose and msgs:
            print("\n".join(msgs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode:
        raise RuntimeError("link failed:\n" + p.stdout + p.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
