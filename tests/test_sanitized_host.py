"""The C-ABI layer's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): api.hip built for the host alone, the kernel launchers replaced by
recording stubs (tests/sanitize/stub_launchers.cpp), and a driver that calls every
entry point with refused and accepted arguments (tests/sanitize/abi_validation.cpp).
Any sanitizer report, or any failed check, fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def test_host_validation_under_address_and_undefined_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "abi_validation")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "masked_verification_attention_amd", "csrc"),
           "-I", SAN]
    # host-only objects: each sanitizer flag sits right after -Xarch_host, so no device code is built with it
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    # api.hip keeps its device part (the allocation-free entry's scratch array), built for gfx950
    # as usual; the stubs and the driver are host code
    jobs = [([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *san, *inc],
             os.path.join(ROOT, "masked_verification_attention_amd", "csrc", "api.hip")),
            ([HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-g", "-std=c++17", *san, *inc],
             os.path.join(SAN, "stub_launchers.cpp")),
            ([HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-g", "-std=c++17", *san, *inc],
             os.path.join(SAN, "abi_validation.cpp"))]
    objs = []
    for cmd, src in jobs:
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        r = subprocess.run([*cmd, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *san, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, \
        r.stdout[-2000:] + r.stderr[-4000:]
    assert "all checks passed" in r.stdout
