"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

csrc/fd_api.cpp (argument checks, the plan, workspace carving) is compiled
with g++ -fsanitize=address,undefined against tests/host/stubs.cpp, which
stands in for the HIP runtime (a 256-CU device) and for the kernel launchers
(nothing runs on a GPU: each launch is checked and recorded; the balanced
split stage walks every share with the kernel's own partition code against
the carved workspace).  Two products:
  - tests/host/host_checks.cpp as an executable: the balanced partition's
    invariants over 2500 seeded ragged batches, the named workloads' plans,
    decode and cascade steps through the stubs;
  - a sanitized libfd.so in place of the real one, against which
    tests/test_abi.py runs in a child process with the sanitizer runtime
    preloaded (every ABI case: exports, heuristic contract, plans,
    validation).
Any sanitizer report fails the run (-fno-sanitize-recover=all, halt on
error).  Builds go to _build/host_sanitized/ (not part of the repository).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "host_sanitized")
CSRC = os.path.join(ROOT, "decode_attention_03_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
FLAGS = ["-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-I" + HOST]
SOURCES = [os.path.join(CSRC, "fd_api.cpp"), os.path.join(HOST, "stubs.cpp")]
ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer")


def _gxx():
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("needs g++ and the HIP headers")
    return gxx


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    out = res.stdout + res.stderr
    return res.returncode, out


@pytest.fixture(scope="module")
def builds():
    gxx = _gxx()
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "host_checks")
    rc, out = _run([gxx, *FLAGS, *SAN, os.path.join(HOST, "host_checks.cpp"), *SOURCES,
                    "-o", exe])
    assert rc == 0, out
    lib = os.path.join(OUT, "libfd.so")
    rc, out = _run([gxx, *FLAGS, *SAN, "-shared", "-fPIC", "-Wl,-Bsymbolic", *SOURCES,
                    "-o", lib])
    assert rc == 0, out
    sys.path.insert(0, ROOT)
    from decode_attention_03_amd import build

    import json

    with open(build.record_path(lib), "w", encoding="utf-8") as f:
        json.dump({"sources_sha256": build.library_source_hash(),
                   "flags": ["host code only, sanitized, stub launchers"]}, f)
    return exe, lib


def test_host_checks_clean_under_sanitizers(builds):
    exe, _ = builds
    rc, out = _run([exe], env=dict(os.environ, **ENV))
    print(out)
    assert rc == 0, out
    assert "host checks passed" in out
    assert not any(r in out for r in REPORTS), out


def test_abi_cases_clean_under_sanitizers(builds):
    """tests/test_abi.py against the sanitized host build, in a child process
    whose first preloaded library is the ASan runtime."""
    _, lib = builds
    gcc = shutil.which("gcc") or "gcc"
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("the ASan runtime is not installed")
    env = dict(os.environ, **ENV)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = asan + (":" + pre if pre else "")
    env["FD_TEST_LIBRARY"] = lib
    rc, out = _run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                    "-q", "-p", "no:cacheprovider", "-m", "not gpu"], env=env, cwd=ROOT)
    print(out[-3000:])
    assert rc == 0, out[-5000:]
    assert not any(r in out for r in REPORTS), out[-5000:]
    assert " passed" in out
