"""The C-ABI argument checks of api.cpp built for the host alone, under AddressSanitizer
and UndefinedBehaviorSanitizer, with stand-in launchers (tests/sanitize/): every entry
point's error paths and valid paths, older struct versions as heap blocks of exactly their
size.  No GPU and no device code are involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")


def hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


def test_abi_checks_under_host_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "abi_checks")
    srcs = [os.path.join(ROOT, "ring_exact_attention_amd", "csrc", "api.cpp"),
            os.path.join(SAN, "stub_launch.cpp"), os.path.join(SAN, "abi_checks.cpp")]
    # host-only compilation: the sanitizers apply to host code (each flag after -Xarch_host)
    cmd = [hipcc(), "-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "ring_exact_attention_amd", "csrc"),
           *srcs, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "checks passed" in run.stdout
