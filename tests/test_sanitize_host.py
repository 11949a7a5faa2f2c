"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Builds, into a temporary directory:
  - the oracle (oracle/oracle.c) with gcc;
  - the library's entry points (pool_stencil_amd/csrc/api.hip) for the host only,
    linked against test stand-ins for the kernel launchers (tests/sanitize/stubs.cpp)
    that record the call and touch no pointer;
  - a driver (tests/sanitize/driver.c) that sweeps the shape queries against the
    oracle's extent functions, walks every entry point's validation paths (including
    the size limits and extreme arguments) and runs the oracle's loops with padding,
    stride and dilation on small tensors.
Every object carries -fsanitize=address,undefined with recovery off, so any
out-of-bounds access, overflow or other undefined behaviour aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def _hipcc():
    p = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return p if os.path.exists(p) else shutil.which("hipcc")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stdout[-2000:] + r.stderr[-4000:])
    return r


def test_host_code_under_sanitizers(tmp_path):
    hipcc = _hipcc()
    if hipcc is None or shutil.which("gcc") is None:
        pytest.skip("hipcc or gcc not available")
    d = str(tmp_path)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "pool_stencil_amd", "csrc")]
    # host-only objects: each sanitizer flag applies to the host side alone
    host_san = [t for f in SAN for t in ("-Xarch_host", f)]
    for src, obj in [("pool_stencil_amd/csrc/api.hip", "api.o"), ("tests/sanitize/stubs.cpp", "stubs.o")]:
        _run([hipcc, "-x", "hip", "--cuda-host-only", "--offload-arch=gfx950", "-O1", "-g",
              "-std=c++17", *host_san, *inc, "-c", os.path.join(ROOT, src), "-o", obj], d)
    _run(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", *SAN, "-c",
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", "oracle.o"], d)
    _run(["gcc", "-O1", "-g", *SAN, *inc, "-c", os.path.join(ROOT, "tests", "sanitize", "driver.c"),
          "-o", "driver.o"], d)
    _run([hipcc, "--offload-arch=gfx950", *host_san, "-fopenmp", "api.o", "stubs.o", "oracle.o",
          "driver.o", "-o", "driver", "-lm"], d)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([os.path.join(d, "driver")], cwd=d, capture_output=True, text=True,
                       env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-6000:]
    assert "sanitize ok" in r.stdout
