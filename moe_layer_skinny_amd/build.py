"""Build libkk.so (the C-ABI library) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkk.so")

SOURCES = ["kk_gemv.hip", "kk_mfma.hip", "kk_scratch.hip", "kk_api.cpp"]
ARCH = "gfx950"
# Packed fp32 instructions are kept out of every kernel.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> tuple[subprocess.Popen, str]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = DEVICE_FLAGS
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(_compile(s), s) for s in SOURCES]
    objs = []
    for (proc, obj), src in jobs:
        out, _ = proc.communicate()
        # hipcc's host pass does not know the device-only feature flag; that note is noise
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if proc.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
        if verbose and lines:
            print("\n".join(lines), file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    subprocess.check_call(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
