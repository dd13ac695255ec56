"""The host side of the C ABI and the CPU oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU).

The argument checks in moe_permute_api.cpp (span and overlap arithmetic in
64-bit products, alignment, workspace sizes) and the launch planner are the
only barrier between a bad caller and a kernel launch on bad pointers, and the
oracle's loops over malloc'd arrays are the reference every parity test
trusts.  This test builds both with ``-fsanitize=address,undefined`` (any
report is fatal): the C ABI against a stub HIP runtime that reports no device
and a stub launch layer that checks what reaches it (tests/sanitize/), the
oracle from its own source.  It then runs the ABI host checks, the planner
checks and the oracle pins against those builds in a child pytest with the
ASan runtime preloaded.  Hosts with a visible GPU skip it (the fake-pointer
ABI checks only run where no kernel can be launched).
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_token_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-fPIC"]


def _gpu_visible() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def _asan_runtime():
    if shutil.which("gcc") is None:
        return None
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


pytestmark = [
    pytest.mark.skipif(_gpu_visible(), reason="the fake-pointer ABI checks run only on a host without a GPU"),
    pytest.mark.skipif(_asan_runtime() is None, reason="gcc with the AddressSanitizer runtime is not available"),
]


def _build(tmp):
    lib = os.path.join(tmp, "libmoe_permute_san.so")
    subprocess.run(["g++", "-std=c++17", "-Wall", *FLAGS, "-shared", "-I", os.path.join(SAN, "stub_include"),
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "moe_permute_api.cpp"),
                    os.path.join(SAN, "launch_stub.cpp"), "-o", lib], check=True)
    orc = os.path.join(tmp, "libmoe_oracle_san.so")
    subprocess.run(["gcc", *FLAGS, "-ffp-contract=off", "-shared", os.path.join(ROOT, "oracle", "moe_oracle.c"),
                    "-lm", "-o", orc], check=True)
    return lib, orc


def test_abi_planner_and_oracle_clean_under_sanitizers(tmp_path):
    lib, orc = _build(str(tmp_path))
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = _asan_runtime() + ((":" + pre) if pre else "")  # the ASan runtime first, nothing removed
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["MOE_TEST_PERMUTE_LIB"] = lib    # tests/conftest.py points the binding at it
    env["MOE_ORACLE_LIB"] = orc          # the oracle loads it instead of its own build
    env["MOE_TEST_SANITIZE_FLAGS"] = " ".join(FLAGS[2:])  # the planner driver compiles with them too
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           "tests/test_abi_host.py", "tests/test_plan_host.py", "tests/test_binding_host.py",
           "tests/test_oracle_pins.py", "tests/test_golden_and_inputs.py"]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]


CANARY = r"""
#include <stdlib.h>
int canary_read_past_end(int n) {
    int* a = (int*)malloc(sizeof(int) * n);
    for (int i = 0; i < n; ++i) a[i] = i;
    int s = a[n];  /* one past the end */
    free(a);
    return s;
}
"""


def test_the_harness_reports_a_heap_overflow(tmp_path):
    """The child environment above does catch a read past a malloc'd block
    (a CPU-only canary built with the same flags), so a clean run means clean."""
    src = tmp_path / "canary.c"
    src.write_text(CANARY)
    so = str(tmp_path / "libcanary.so")
    subprocess.run(["gcc", *FLAGS, "-shared", str(src), "-o", so], check=True)
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = _asan_runtime() + ((":" + pre) if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    code = "import ctypes, sys; print(ctypes.CDLL(sys.argv[1]).canary_read_past_end(5))"
    res = subprocess.run([sys.executable, "-c", code, so], env=env, capture_output=True, text=True, timeout=120)
    assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr, res.stderr[-2000:]
