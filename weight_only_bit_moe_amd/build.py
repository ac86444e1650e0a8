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


# Host-side sanitizer build: the C ABI's host code (api.hip) and the oracle's C
# code instrumented with AddressSanitizer and UndefinedBehaviorSanitizer, linked
# with the other library objects into tests/sanitize/host_check (no GPU needed).
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
SAN_DRIVER = os.path.join(ROOT, "tests", "sanitize", "host_check.cpp")
SAN_EXE = os.path.join(ROOT, "tests", "sanitize", "host_check")


def build_sanitized(verbose: bool = False) -> str:
    """Build tests/sanitize/host_check; returns its path."""
    llvm = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin")
    clang = os.path.join(llvm, "clang")
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(bdir, src + ".o")
        if src == "api.hip":
            obj = os.path.join(bdir, "api.san.o")
            # device code as usual; every sanitizer flag applies to the host pass only
            host = [f for flag in SAN for f in ("-Xarch_host", flag)]
            _run([hipcc()] + flags() + host + ["-g", "-c", os.path.join(CSRC, src), "-o", obj],
                 verbose)
        elif not os.path.exists(obj):
            _run([hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    oracle_obj = os.path.join(bdir, "moe_oracle.san.o")
    _run([clang, "-std=c99", "-O1", "-g", "-fPIC"] + SAN +
         ["-c", os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", oracle_obj], verbose)
    driver_obj = os.path.join(bdir, "host_check.san.o")
    _run([clang + "++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__",
          "-I", "/opt/rocm/include", "-I", INCLUDE] + SAN +
         ["-c", SAN_DRIVER, "-o", driver_obj], verbose)
    _run([clang + "++"] + SAN + ["-o", SAN_EXE, driver_obj, oracle_obj] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lm"], verbose)
    return SAN_EXE


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    text = "\n".join(l for l in r.stdout.decode(errors="replace").splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{text}")


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
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose=True))
    else:
        print(build(verbose=True))
