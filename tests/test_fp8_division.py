"""The FP8 quantization's division shortcut gives the codes of the correctly
rounded division (see tests/fp8_division_check.c): compiled with gcc and run
over every bf16 scale magnitude that takes the shortcut and every bf16
activation value."""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the check")
def test_fp8_division_shortcut_codes(tmp_path):
    exe = str(tmp_path / "fp8_division_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-o", exe,
                    os.path.join(HERE, "fp8_division_check.c"), "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(16, os.cpu_count() or 1)))
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    scales, values, differ = (int(t) for t in re.findall(r"\d+", r.stdout)[:3])
    assert differ == 0 and scales > 25000 and values > 10 ** 9, r.stdout
