"""Build libfca.so (HIP, gfx950) in-tree with hipcc.

    python -m shared_prefix_kv_amd.build

Every .hip file under csrc/ is compiled (hipcc, gfx950) and every .cpp file
(host-only code, the planner) is compiled with the host compiler, to
objects in _build/ that are linked into shared_prefix_kv_amd/libfca.so.  Packed fp32 instructions are turned
off for device code (``-packed-fp32-ops``); hipcc's host pass warns that it
does not know that feature, which is harmless.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfca.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
    # The leading pointer arguments of the kernels arrive in scalar registers.
    "-mllvm",
    "-amdgpu-kernarg-preload-count=16",
    "-I" + os.path.join(ROOT, "include"),
]


HOST_CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wextra", "-Wno-unused-parameter", "-I" + os.path.join(ROOT, "include")]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):
        cmd = [HOST_CXX, *HOST_FLAGS, "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        line
        for line in (res.stdout + res.stderr).splitlines()
        if "packed-fp32-ops" not in line  # host-pass notice about the device-only feature
    )
    if res.returncode != 0:
        raise RuntimeError(f"{cmd[0]} failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libfca.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
