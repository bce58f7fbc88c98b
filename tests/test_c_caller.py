"""The C ABI from plain C: tests/host/c_caller.c includes include/aah_attn.h as C99 and links
libaah_attn.so, with no Python, no torch and no C++ in the caller.

On the CPU it runs the argument checks (ABI version, a NULL tensor refused before any HIP call, an empty
problem accepted with NULL tensors, status strings, a workspace size).  On the GPU (--device) it allocates
with the HIP runtime's C API, runs forward and backward in bf16 and fp32 on a stream it creates, and checks
closed forms of the windowed softmax ("Asymmetric Attention Heads" section 5.8): a window of 1 returns V and
LSE = scale q.k, its dV equals dO, and constant V rows give O = that row for any window.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "head_causal_local_amd")


def _build(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    if not os.path.exists(os.path.join(PKG, "libaah_attn.so")):
        pytest.fail("libaah_attn.so is not built (python -m head_causal_local_amd.build)")
    exe = tmp_path / "c_caller"
    subprocess.run(["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "host", "c_caller.c"), "-o", str(exe),
                    "-L", PKG, "-Wl,-rpath," + PKG, "-laah_attn", "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib",
                    "-lamdhip64", "-lm"], check=True, timeout=120)
    return exe


def test_c_caller_argument_checks(tmp_path):
    exe = _build(tmp_path)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "ok"


@pytest.mark.gpu
def test_c_caller_on_device(tmp_path):
    exe = _build(tmp_path)
    print("c_caller --device", flush=True)
    res = subprocess.run([str(exe), "--device"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "ok"
