"""Host-only build of the library under AddressSanitizer and UndefinedBehaviorSanitizer.

The C ABI layer (argument checking, work-list caches) and the planner are plain host C++.  Here they are
compiled by g++ with -fsanitize=address,undefined, linked against kernel-launch stubs
(tests/host/launch_stubs.cpp: every launch reports that no device is present, as on this machine), and the
CPU tests of argument checking and planning (test_abi_cpu.py, test_planner.py, test_split_planner.py) run
against that library in a subprocess with the sanitizer runtimes preloaded; any report aborts the run.  The
work-list cache's bookkeeping (plan_cache.hpp) has its own C++ unit test, built the same way.

By hand (repository root):
    g++ -std=c++17 -O1 -g -fPIC -shared -fsanitize=address,undefined -fno-sanitize-recover=all \\
        -D__HIP_PLATFORM_AMD__ -I /opt/rocm/include -I include -I head_causal_local_amd/csrc \\
        head_causal_local_amd/csrc/workplan.cpp head_causal_local_amd/csrc/aah_api.cpp tests/host/launch_stubs.cpp \\
        -L/opt/rocm/lib -Wl,-rpath,/opt/rocm/lib -lamdhip64 -o /tmp/libaah_host.so
    LD_PRELOAD="$(g++ -print-file-name=libasan.so) $(g++ -print-file-name=libubsan.so)" \\
        ASAN_OPTIONS=detect_leaks=0 AAH_TEST_HOST_LIB=/tmp/libaah_host.so \\
        python -m pytest tests/test_abi_cpu.py tests/test_planner.py tests/test_split_planner.py -m "not gpu"
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "head_causal_local_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _need_toolchain():
    if shutil.which("g++") is None:
        pytest.skip("g++ is not installed")
    if _runtime("libasan.so") is None or _runtime("libubsan.so") is None:
        pytest.skip("g++ has no sanitizer runtimes")


def test_plan_cache_lru_unit(tmp_path):
    """The cache never holds more than its capacity over thousands of distinct window vectors, evicts the
    least recently used unpinned entry, and keeps pinned ones (tests/host/plan_lru_test.cpp)."""
    _need_toolchain()
    exe = tmp_path / "plan_lru_test"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", *SAN, "-I", CSRC,
                    os.path.join(ROOT, "tests", "host", "plan_lru_test.cpp"), "-o", str(exe)], check=True,
                   timeout=300)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "ok"


def test_validation_and_planner_clean_under_sanitizers(tmp_path):
    _need_toolchain()
    if not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("the HIP runtime library is not installed")
    lib = tmp_path / "libaah_host.so"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "workplan.cpp"), os.path.join(CSRC, "aah_api.cpp"),
           os.path.join(ROOT, "tests", "host", "launch_stubs.cpp"),
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", str(lib)]
    subprocess.run(cmd, check=True, timeout=600, capture_output=True)
    syms = subprocess.run(["nm", "-D", str(lib)], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms  # the library really is instrumented
    env = dict(os.environ)
    env.update(LD_PRELOAD=f"{_runtime('libasan.so')} {_runtime('libubsan.so')}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               AAH_TEST_HOST_LIB=str(lib))
    tests = [os.path.join(ROOT, "tests", t) for t in ("test_abi_cpu.py", "test_planner.py", "test_split_planner.py")]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                          *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out
