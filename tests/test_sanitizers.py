"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer:

- the C ABI's host-side argument checks and kernel selection
  (csrc/dsa_abi.cpp + csrc/envelopes.cpp) with the kernel launches stubbed
  out (tests/sanitize/abi_host_check.cpp), called with valid, invalid and
  extreme sizes;
- the oracle (oracle/dsa_oracle.c), driven through its Python wrapper on
  small inputs and edge cases (tests/sanitize/oracle_drive.py).

Host code only: built with g++/gcc, no device code, nothing touches a GPU.
Any sanitizer report aborts the program (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_scores_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-O1", "-g"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, (f"{' '.join(cmd)} exited {r.returncode}\n"
                               f"stdout:\n{r.stdout[-4000:]}\nstderr:\n{r.stderr[-8000:]}")
    return r


def test_abi_host_checks_under_asan_ubsan(tmp_path):
    _need("g++")
    exe = str(tmp_path / "abi_host_check")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
          os.path.join(CSRC, "dsa_abi.cpp"), os.path.join(CSRC, "envelopes.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp"), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env)
    assert " 0 failures" in r.stdout, r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    _need("gcc")
    lib = str(tmp_path / "libdsa_oracle_san.so")
    _run(["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp", *SAN, "-o", lib,
          os.path.join(ROOT, "oracle", "dsa_oracle.c"), "-lm"])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan.so not found")
    # the Python interpreter itself is not instrumented: leaks are not checked
    env = dict(os.environ, LD_PRELOAD=asan, DSA_ORACLE_LIB=lib, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "oracle_drive.py")],
             env=env)
    assert "oracle drive: done" in r.stdout, r.stdout
