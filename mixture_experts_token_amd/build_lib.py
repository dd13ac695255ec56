"""Compile the HIP library ``libmoe_permute.so`` for gfx950, in-tree.

    python -m mixture_experts_token_amd.build_lib

Each source is compiled to its own object (in parallel, under ``_build/``)
and the objects are linked into the shared library.  Packed fp32 instructions
are switched off for every HIP source
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns
that it does not know the feature, which is harmless.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_permute.so")
PROBE_LIB = os.path.join(PKG, "libhbm_probe.so")

SOURCES = ["moe_permute_wave.hip", "moe_permute_fused.hip", "moe_permute_coarse.hip", "moe_permute_staged.hip",
           "moe_permute_rows.hip", "moe_permute_launch.hip", "moe_unpermute.hip", "moe_quant_kernels.hip", "moe_gemm_kernels.hip", "moe_gemm_skinny.hip", "moe_permute_api.cpp"]
HEADERS = ["moe_launch.h", "moe_plan.h", "moe_permute_device.h", "moe_gemm_device.h"]
PROBE_SOURCES = ["hbm_probe.hip"]  # streaming-ceiling kernels used by bench.py only

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
NOISE = "packed-fp32-ops"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, csrc: str = CSRC, lib: str = LIB, probe_lib: str | None = PROBE_LIB,
          obj_dir: str = OBJ_DIR) -> str:
    """Compile every source (always, also when a built library is present) and link."""
    jobs = [(lib, SOURCES)] + ([(probe_lib, PROBE_SOURCES)] if probe_lib else [])
    objs = {}
    work = []
    for target, sources in jobs:
        tag = os.path.splitext(os.path.basename(target))[0]
        objs[target] = []
        for s in sources:
            obj = os.path.join(obj_dir, "%s.%s.o" % (tag, os.path.splitext(s)[0]))
            objs[target].append(obj)
            work.append((os.path.join(csrc, s), obj, csrc))
    os.makedirs(obj_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(work))) as pool:
        for msg in pool.map(lambda w: _compile(*w, verbose=verbose), work):
            if msg:
                print(msg, flush=True)
    for target, _ in jobs:
        _link(target, objs[target], verbose)
    return lib


def _run(cmd, verbose: bool, what: str) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if NOISE not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("%s failed:\n%s" % (what, "\n".join(msgs)))
    return "\n".join(msgs) if verbose else ""


def _compile(src: str, obj: str, csrc: str, verbose: bool) -> str:
    tmp = obj + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", csrc, "-c", "-o", tmp, src]
    out = _run(cmd, verbose, "hipcc -c %s" % os.path.basename(src))
    os.replace(tmp, obj)
    return out


def _link(target: str, objs, verbose: bool) -> None:
    tmp = target + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    out = _run(cmd, verbose, "link %s" % os.path.basename(target))
    if out:
        print(out, flush=True)
    os.replace(tmp, target)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
