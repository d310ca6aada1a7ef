"""Build libgdn.so (hand-written HIP for gfx950) in-tree with hipcc.

Each .hip file under csrc/ is compiled to an object in parallel, then linked
into gated_deltanet_recurrence_delta_amd/libgdn.so.  Always rebuilds.
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
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"),
    # Keep the compiler from forming packed-fp32 (v_pk_*_f32) instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Options for single files.  gemm.hip: matrix-core instructions in their
# VGPR form, so its 128 accumulators per lane are not shuffled between
# accumulation and vector registers.
FILE_FLAGS = {
    "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = ([HIPCC] + FLAGS + FILE_FLAGS.get(os.path.basename(src), [])
           + ["-c", src, "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout,
                                                            r.stderr))
    return obj


def build(verbose: bool = True) -> str:
    t0 = time.time()
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC",
                        "-o", tmp] + objs, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    # A kernel whose host launch stub the host pass dropped links fine and
    # only fails when the library is loaded; refuse such a library here.
    r = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True,
                       text=True)
    stubs = [l.split()[-1] for l in r.stdout.splitlines() if "__device_stub__" in l]
    if stubs:
        os.remove(tmp)
        raise RuntimeError("undefined kernel launch stubs: %s" % ", ".join(stubs))
    os.replace(tmp, LIB)
    if verbose:
        print("built %s in %.1fs" % (LIB, time.time() - t0), file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
