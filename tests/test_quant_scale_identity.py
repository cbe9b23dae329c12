"""Host check of an arithmetic identity the quantizer kernels rely on.

The kernels compute the block scale d = amax / 127 without a division:
q0 = f32(amax * R) with R = f32(1/127), then one fma-corrected step. That this
equals the IEEE quotient for every non-negative finite f32 is checked here by
enumeration, compiled with gcc (IEEE fma, no contraction, no denormal flush).
"""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_scale_without_division_matches_ieee_quotient():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "q_scale_check")
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                        os.path.join(HERE, "q_scale_check.c"), "-o", exe, "-lm"], check=True)
        env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
        assert r.returncode == 0, r.stdout + r.stderr
        assert r.stdout.strip() == "mismatches 0"
