"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, gcc) runs every entry point on small and edge-case shapes
(tests/oracle_sanitize_main.c) without a report: no read or write outside a
buffer, no leak, no undefined arithmetic."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_main.c"),
           "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("this gcc has no sanitizer runtime: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stderr[-4000:]
    assert "clean" in run.stdout
