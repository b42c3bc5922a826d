"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (gcc): a C driver
(tests/oracle_sanitize.c) runs every oracle entry point on thousands of small random inputs;
any out-of-bounds access, leak or undefined operation fails the run.  The parity tests trust
the oracle, so its memory safety is checked on its own."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not installed")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fopenmp", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(HERE, "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip("this gcc has no sanitizer runtime: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0 and "ok" in run.stdout, (run.stdout[-2000:], run.stderr[-4000:])
