"""The quantiser's division shortcut (one reciprocal and one fused residual correction per
element, used for scales in [2^-32, 2^32]) yields the IEEE float32 quotient for every BF16
significand against every float32 scale significand, and the same E4M3FN codes as IEEE division
for every BF16 pattern over that scale range (tests/host/recip_division.c). Planted mistakes
(no correction step, no overflow guard, no sign fix) each fail it. CPU only: the check is of the
arithmetic identity; the GPU insert tests compare the kernel's bytes with the oracle."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_residual_division_is_exact(tmp_path):
    exe = str(tmp_path / "recip_division")
    src = os.path.join(HERE, "host", "recip_division.c")
    # -ffp-contract=off: x * r must round on its own; -fno-fast-math keeps IEEE division
    r = subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", src, "-o", exe, "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env.setdefault("OMP_NUM_THREADS", str(min(8, os.cpu_count() or 1)))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout
