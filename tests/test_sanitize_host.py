"""The library's host side and the CPU oracle under AddressSanitizer and
UndefinedBehaviorSanitizer.

Builds, with ROCm's clang and no device code: the C ABI layer (abi.hip,
host pass only), the launch planning (plan.cpp), stand-ins for the kernel
launchers (tests/sanitize/launch_stubs.cpp), the oracle (oracle/dsa_oracle.c,
single-threaded) and a driver (tests/sanitize/host_driver.c) that walks every
entry point's error paths and valid calls down to their launches, the size
queries over small and very large shapes, the layer plan and the frequencies,
then the oracle on tiny inputs.  Any sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_12_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
LLVM = "/opt/rocm/llvm/bin"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not os.path.exists(os.path.join(LLVM, "clang++")), reason="ROCm clang not installed")
def test_host_paths_and_oracle_clean_under_sanitizers(tmp_path):
    d = str(tmp_path)
    clang, clangxx = os.path.join(LLVM, "clang"), os.path.join(LLVM, "clang++")
    # the C ABI layer, host pass only (no device code, no code object);
    # each sanitizer flag goes to the host pass alone
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    _run([HIPCC, "--offload-host-only", "-x", "hip", "-std=c++17", "-fPIC", *host_san, "-c",
          os.path.join(CSRC, "abi.hip"), "-o", "abi.o"], d)
    _run([HIPCC, "--offload-host-only", "-x", "hip", "-std=c++17", "-fPIC", *host_san, "-c",
          os.path.join(HERE, "launch_stubs.cpp"), "-o", "stubs.o"], d)
    _run([clangxx, "-std=c++17", *SAN, "-c", os.path.join(CSRC, "plan.cpp"), "-o", "plan.o"], d)
    _run([clang, "-std=c11", *SAN, "-Wno-unknown-pragmas", "-c", os.path.join(ROOT, "oracle", "dsa_oracle.c"),
          "-o", "oracle.o"], d)
    _run([clang, "-std=c11", *SAN, "-c", os.path.join(HERE, "host_driver.c"), "-o", "driver.o"], d)
    _run([clangxx, *SAN, "abi.o", "stubs.o", "plan.o", "oracle.o", "driver.o", "-o", "host_driver", "-lm"], d)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([os.path.join(d, "host_driver")], cwd=d, capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    assert "clean under the sanitizers" in r.stdout
