"""Build steps for the native parts of the package.

- libdsa3d.so: the HIP kernels and the C ABI (include/dsa3d.h), gfx950 only.
- synth/libdsa3d_synth.so: the seeded input generator (plain C + OpenMP).

Every call compiles from source; nothing is cached between calls.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdsa3d.so")
SYNTH_SRC = os.path.join(PKG, "synth", "synth.c")
SYNTH_LIB = os.path.join(PKG, "synth", "libdsa3d_synth.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of the device code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
    "-I" + CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return out


def hip_sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build_lib(extra_flags=()):
    objs = []
    srcs = hip_sources()
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)

    def one(src):
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        _run([HIPCC, *HIP_FLAGS, *extra_flags, "-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def build_synth():
    tmp = SYNTH_LIB + ".tmp"
    _run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", SYNTH_SRC, "-o", tmp, "-lm"])
    os.replace(tmp, SYNTH_LIB)
    return SYNTH_LIB


def build_all():
    build_synth()
    build_lib()
