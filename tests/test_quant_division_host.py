"""Exhaustive host check of the bf16 quotient in the quantise kernels.

The kernels quantise bf16 x as the E4M3FN code of x / scale (the per-token
activation quantisation of vLLM PR #19636, "[Kernels] MoE refactor",
highlights) without a division per element: a correctly rounded reciprocal
and the FMA correction step of Markstein's division.  `quant_division_check.c`
runs every positive finite bf16 amax (scale = amax / 448 in [2^-100, 2^126])
against every finite bf16 x with |x| <= amax and requires the quotient that
decides the code to be the correctly rounded one.  The GPU parity tests then
compare the kernels' codes with the oracle's.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_bf16_quotient_exhaustive(tmp_path):
    exe = str(tmp_path / "quant_division_check")
    base = ["gcc", "-O2", "-mfma", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "quant_division_check.c"), "-lm"]
    if subprocess.run(base[:1] + ["-fopenmp"] + base[1:], capture_output=True).returncode != 0:
        subprocess.run(base, check=True, capture_output=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout[-2000:]
    assert "failures 0" in out.stdout
    # every positive finite bf16 amax whose float scale lies in the checked range
    amax = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    scale = amax / np.float32(448.0)
    expected = int(np.count_nonzero((scale >= np.float32(2.0**-100)) & (scale <= np.float32(2.0**126))))
    assert int(out.stdout.split("scales ")[1].split()[0]) == expected > 28000
