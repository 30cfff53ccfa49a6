"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_driver.c calls every oracle entry point on small seeded
inputs; it is built here together with oracle/nystrom_oracle.c by gcc with
-fsanitize=address,undefined (host code only; nothing of the GPU library is
involved) and must run to the end with no sanitizer report and no leak.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build(tmp):
    exe = os.path.join(tmp, "oracle_sanitized")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-static-libasan",
           os.path.join(ROOT, "oracle", "nystrom_oracle.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"), "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return exe, r


def test_oracle_runs_clean_under_asan_and_ubsan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        exe, r = _build(tmp)
        if r.returncode != 0 and ("libasan" in r.stderr or "libubsan" in r.stderr):
            pytest.skip("gcc sanitizer runtimes not installed: " + r.stderr[-300:])
        assert r.returncode == 0, r.stderr
        # the ASan runtime is linked statically, so it needs no place in the
        # dynamic library list
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        report = run.stdout + run.stderr
        assert run.returncode == 0, report[-4000:]
        assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
        assert "all paths ran" in run.stdout
