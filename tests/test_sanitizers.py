"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

- tests/sanitize/oracle_driver.c runs every oracle routine on small inputs in
  exactly sized heap buffers, built with gcc and both sanitizers;
- tests/sanitize/abi_driver.cpp calls every C entry point with invalid
  arguments and with n = 0 against a library build whose host code carries both
  sanitizers (device code is built normally); validation runs before any HIP
  call, so no GPU is needed.
"""
import os
import subprocess
import tempfile

import pytest

from gradient_sync_amd import _build as B

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, (cmd[0], p.stdout[-2000:], p.stderr[-4000:])
    return p.stdout


def test_oracle_under_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_driver")
        run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer",
             os.path.join(ROOT, "oracle", "dp_oracle.c"),
             os.path.join(HERE, "sanitize", "oracle_driver.c"), "-o", exe, "-lm"])
        out = run([exe], env=ENV, timeout=300)
        assert "0 failures" in out


@pytest.mark.timeout(900)
def test_library_host_code_under_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        inc = ["-I", B.CSRC, "-I", os.path.join(ROOT, "include")]
        host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all"]
        procs, objs = [], []
        for src in B.SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [B.HIPCC, f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
                   "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
                   "-packed-fp32-ops", *host_san, *inc, "-c", os.path.join(B.CSRC, src),
                   "-o", obj]
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.DEVNULL,
                                                stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        for src, p in procs:
            _, err = p.communicate()
            assert p.returncode == 0, (src, err[-3000:])
        drv = os.path.join(tmp, "abi_driver.o")
        run(["/opt/rocm/llvm/bin/clang++", "-O1", "-g", "-std=c++17",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", *inc[2:], "-c",
             os.path.join(HERE, "sanitize", "abi_driver.cpp"), "-o", drv])
        exe = os.path.join(tmp, "abi_driver")
        run([B.HIPCC, f"--offload-arch={B.ARCH}", *host_san[:4], *objs, drv, "-o", exe])
        out = run([exe], env=ENV, timeout=120)
        assert "0 failures" in out
