"""Build the gfx950 shared library libmoe_wna16.so in-tree with hipcc.

    python -m weight_only_bit_moe_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_wna16.so")
SOURCES = ["kernels.hip", "quantize.hip", "prepare.hip", "api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-Wno-unused-function",
        # packed FP32 VALU forms stay off (ordinary float code, no v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def build(verbose: bool = False, jobs: int = 3) -> str:
    """Compile every source to an object in parallel, then link the library."""
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(bdir, src + ".o")
        objs.append(obj)
        cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _drain(procs)
    _drain(procs)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _drain(procs):
    while procs:
        cmd, p = procs.pop(0)
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-FP32 feature name: harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            raise RuntimeError(f"build failed: {' '.join(cmd)}\n{text}")
        if text.strip():
            print(text, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
