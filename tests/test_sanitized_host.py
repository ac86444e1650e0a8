"""The host code of the C ABI (argument checks, workspace layout, tiling plan)
and the oracle's C code, built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU (tests/sanitize/host_check.cpp;
`python -m weight_only_bit_moe_amd.build --sanitize`).  No call in it reaches
the device."""
import os
import subprocess

from weight_only_bit_moe_amd import build as B


def test_host_code_clean_under_sanitizers():
    exe = B.build_sanitized()
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("host checks passed")
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
