"""The library's host code (argument checks, workspace queries, plan arithmetic)
and the oracle under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

tests/sanitize/host_checks.cpp calls every qg_check_* twin and workspace query
over valid and invalid shapes (fake device addresses: the twins never
dereference them and launch nothing) and every oracle function on small
inputs.  The HIP sources are built with the sanitizers on their host side only
(-Xarch_host); the device code is built as usual and never runs here.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from bit_quantized_decode_group_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stdout + r.stderr)


@pytest.mark.skipif(not (os.path.exists(B.HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers missing")
def test_host_code_and_oracle_under_asan_and_ubsan(tmp_path):
    hip_flags = [f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
                 "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
    for f in SAN:
        hip_flags += ["-Xarch_host", f]
    jobs = [[B.HIPCC, *hip_flags, "-c", os.path.join(B.CSRC, s), "-o", str(tmp_path / (s + ".o"))]
            for s in B.SOURCES]
    jobs.append([CLANG, "-O1", "-g", "-std=c11", "-ffp-contract=off", *SAN, "-c",
                 os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(tmp_path / "oracle.o")])
    jobs.append([CLANGXX, "-O1", "-g", "-std=c++17", *SAN, "-c",
                 os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), "-o", str(tmp_path / "host_checks.o")])
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        list(ex.map(_run, jobs))
    exe = str(tmp_path / "host_checks")
    objs = [str(tmp_path / (s + ".o")) for s in B.SOURCES] + [str(tmp_path / "oracle.o"),
                                                             str(tmp_path / "host_checks.o")]
    _run([CLANGXX, *SAN, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "host checks:" in out and "oracle status 0" in out, out[-2000:]
