"""The seeded input generator and the CPU oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only): tests/sanitize_driver.c drives
every oracle entry point on a tiny generated layer; any out-of-bounds access,
leak or undefined operation aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    cmd = ["gcc", "-O1", "-g", "-fopenmp", "-std=c11", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", "-ffp-contract=off",
           os.path.join(ROOT, "tests", "sanitize_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(ROOT, "synth", "synth.c"), "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
