"""Build libmoe.so (the HIP library behind include/moe.h) for gfx950 with hipcc, in-tree.

    python -m sparse_moe_routing_amd.build

Every .hip file under csrc/ is compiled to an object in _build/ (in parallel), then linked into
sparse_moe_routing_amd/libmoe.so. Packed fp32 instructions are disabled for all device code.
The benchmark's streaming-read calibration kernel (probe/read_probe.hip) is built next to it as
libmoe_probe.so, a library of its own: libmoe.so does not contain or call it.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
PROBE_SRC = os.path.join(PKG, "probe", "read_probe.hip")
PROBE_LIB = os.path.join(PKG, "libmoe_probe.so")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def compile_flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wextra", "-Wno-unused-parameter", "-Werror",
            "-I" + os.path.join(ROOT, "include")]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")

    def one(src):
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        cmd = [cc, *compile_flags(), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = (r.stdout + r.stderr)
        # hipcc's host pass does not know the packed-fp32 feature name: that warning is harmless
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + f".tmp{os.getpid()}"
    cmd = [cc, *compile_flags(), "-shared", "-o", tmp, PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n" + r.stdout + r.stderr)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
