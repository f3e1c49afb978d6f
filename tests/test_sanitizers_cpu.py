"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built here and must run clean:
  * the fp64 oracle (oracle/gqa_oracle.c, with OpenMP) driven on small seeded
    problems by tests/sanitize/oracle_check.c, which also checks properties
    the definition fixes (probability rows sum to 1 and reproduce the output
    row, an exact two-shard merge, E4M3 anchors, rejection of a bad problem);
  * the C ABI's host layer (causal_grouped_query_amd/csrc/api.hip compiled as
    plain C++ against tests/sanitize/fakehip and stub launchers), driven by
    tests/sanitize/api_check.cpp through every exported entry point with
    valid and invalid arguments; nothing reaches a GPU.
Any sanitizer report aborts the program (no recovery), failing the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed for the host build")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-std=c11", *FLAGS, "-fopenmp", os.path.join(ROOT, "oracle", "gqa_oracle.c"),
          os.path.join(SAN, "oracle_check.c"), "-o", exe, "-lm"])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", OMP_NUM_THREADS="2"))
    assert "oracle checks passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(CLANG), reason="clang++ is needed for the host build of the C ABI layer")
def test_api_host_layer_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "api_check")
    inc = ["-I" + os.path.join(SAN, "fakehip"), "-I" + SAN, "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "causal_grouped_query_amd", "csrc")]
    _run([CLANG, "-std=c++17", *FLAGS, *inc, "-x", "c++", os.path.join(ROOT, "causal_grouped_query_amd", "csrc",
                                                                        "api.hip"),
          "-x", "none", os.path.join(SAN, "stub_launch.cpp"), os.path.join(SAN, "api_check.cpp"), "-o", exe])
    r = _run([exe], env=ENV)
    assert "api checks passed" in r.stdout
