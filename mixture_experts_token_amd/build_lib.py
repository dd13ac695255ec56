"""Compile the HIP library ``libmoe_permute.so`` for gfx950, in-tree.

    python -m mixture_experts_token_amd.build_lib

Packed fp32 instructions are switched off for every HIP source
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns
that it does not know the feature, which is harmless.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_permute.so")
PROBE_LIB = os.path.join(PKG, "libhbm_probe.so")

SOURCES = ["moe_permute_kernels.hip", "moe_quant_kernels.hip", "moe_gemm_kernels.hip", "moe_permute_api.cpp"]
HEADERS = ["moe_launch.h", "moe_plan.h"]
PROBE_SOURCES = ["hbm_probe.hip"]  # streaming-ceiling kernels used by bench.py only

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    _build_one(PROBE_LIB, PROBE_SOURCES, verbose)
    return _build_one(LIB, SOURCES, verbose)


def _build_one(target: str, sources, verbose: bool) -> str:
    tmp = target + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp,
           *[os.path.join(CSRC, s) for s in sources]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
