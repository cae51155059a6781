"""The CPU oracle (oracle/oracle.c) and the input generator (synth/synth.c) built with the
address and undefined-behaviour sanitizers (gcc, host code only) and run over every
function on small shapes by tests/sanitize_driver.c: no sanitizer report, and the
driver's exact checks hold."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fopenmp", "-ffp-contract=off",
           os.path.join(ROOT, "tests", "sanitize_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(ROOT, "synth", "synth.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "sanitize driver: ok" in r.stdout
