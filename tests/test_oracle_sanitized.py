"""The C oracle built with the address and undefined-behaviour sanitizers
(gcc, host code only) and driven through every entry point on small seeded
problems (tests/oracle_sanitize_driver.c): no out-of-bounds access, leak or
undefined behaviour, in one thread and in several."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "kda_oracle.c")
DRIVER_C = os.path.join(ROOT, "tests", "oracle_sanitize_driver.c")
N_SHAPES = 6


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    build = subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined",
                            "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                            "-fopenmp", ORACLE_C, DRIVER_C, "-o", exe, "-lm"],
                           capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip("the sanitizer runtimes are not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-3000:]
    for threads in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=threads,
                   ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        run = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
        assert run.returncode == 0, run.stderr[-3000:]
        assert "AddressSanitizer" not in run.stderr and "runtime error" not in run.stderr, run.stderr[-3000:]
        assert run.stdout.count(" ok ") == N_SHAPES, run.stdout
