"""Every oracle pin, run against oracle/oracle.c built with AddressSanitizer
and UndefinedBehaviorSanitizer (errors fatal), in a child process that loads
the sanitizer runtime first. An out-of-bounds access, a use of freed memory,
a signed overflow, a misaligned access or a bad shift anywhere the pins reach
in the oracle ends the child with an error."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_pins_under_asan_and_ubsan(tmp_path):
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("gcc has no AddressSanitizer runtime")
    so = str(tmp_path / "liboracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                    SRC, "-o", so, "-lm"], check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(x for x in (libasan, env.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    code = ("import sys\n"
            f"sys.path.insert(0, {ROOT!r})\n"
            "import oracle\n"
            "from tests import oracle_pins as pins\n"
            f"lib = oracle.load({so!r})\n"
            "names = []\n"
            "for name, check in pins.all_checks():\n"
            "    check(lib)\n"
            "    names.append(name)\n"
            "print('pins passed:', len(names))\n")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    assert r.returncode == 0, f"sanitized oracle failed (rc {r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
    assert "pins passed:" in r.stdout
    print(r.stdout.strip().splitlines()[-1])
