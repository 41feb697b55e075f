"""The float64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and run on small inputs through every exported
function (tests/oracle_sanitize.c): no out-of-bounds access, leak,
use-after-free, signed overflow or other undefined behaviour."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "sdm_oracle.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize.c"), "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = {**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
           "UBSAN_OPTIONS": "print_stacktrace=1", "OMP_NUM_THREADS": "3"}
    r = subprocess.run([str(exe)], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
