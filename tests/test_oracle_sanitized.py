"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code, gcc), driven through every function by oracle_sanitize_driver.c
on exactly sized buffers (CPU only).  Built without OpenMP, so the loops run
serially and every access is checked."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "dsc_oracle.c"),
           os.path.join(HERE, "oracle_sanitize_driver.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle calls ok" in r.stdout
    assert "runtime error" not in r.stderr
