"""The CPU oracle and the input generator built with gcc's address and
undefined-behaviour sanitizers, driven over small ragged inputs of every
oracle function (tests/sanitize_driver.c). Any out-of-bounds access, leak or
undefined operation makes the run fail."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    exe = tmp_path / "sanitized"
    srcs = [os.path.join(ROOT, "tests", "sanitize_driver.c"), os.path.join(ROOT, "oracle", "qsa_oracle.c"),
            os.path.join(ROOT, "gen", "qsa_gen.c")]
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-ffp-contract=off", "-o", str(exe), *srcs, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized run done" in r.stdout
